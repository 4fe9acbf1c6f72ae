"""Oracle: sort (token, expert) pairs by expert and pad each segment
(test infrastructure; see ``oracle/__init__.py``).

[MSG] "fused MoE" (moe_align_block_size): the pairs are the entries of the
flattened topk_ids; pair i belongs to expert topk_ids.flat[i].  Pairs are
grouped by expert in ascending expert order, keeping ascending pair order
inside a group (the page uses a stable argsort), and each group is padded
with the placeholder value num_pairs up to a multiple of block_m.  Experts
with no pair get no block.  One expert id is emitted per block_m entries.
"""

import numpy as np


def moe_align_block_size(topk_ids, num_experts, block_m):
    """Returns (sorted_ids int64 [total], expert_ids int64 [total // block_m],
    total).  Written as a loop over experts, appending each expert's pair
    indices in ascending order followed by its padding."""
    flat = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    num_pairs = flat.size
    if block_m < 1:
        raise ValueError("block_m must be positive")
    if num_pairs and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    sorted_ids = []
    expert_ids = []
    for e in range(num_experts):
        members = np.flatnonzero(flat == e)  # ascending pair indices
        if members.size == 0:
            continue
        seg = [int(i) for i in members]
        while len(seg) % block_m != 0:
            seg.append(num_pairs)
        sorted_ids.extend(seg)
        expert_ids.extend([e] * (len(seg) // block_m))
    total = len(sorted_ids)
    return (np.array(sorted_ids, dtype=np.int64),
            np.array(expert_ids, dtype=np.int64), total)


def align_max_padded(num_pairs, num_experts, block_m):
    """Upper bound of the padded total: every non-empty expert adds at most
    block_m - 1 placeholders, and at most min(E, pairs) experts are
    non-empty; rounded up to a whole block.  It is reached when E >= pairs
    (every pair alone) or when pairs - E is a multiple of block_m (every
    expert holds 1 mod block_m pairs); otherwise the true maximum is lower."""
    bound = num_pairs + min(num_experts, num_pairs) * (block_m - 1)
    return -(-bound // block_m) * block_m
