"""Seeded generators (input preparation only)."""

import numpy as np


def host_rng(config_id, tensor_id, sub_id=0):
    """PCG64 stream for one tensor (or one expert's slab of it)."""
    return np.random.default_rng([int(config_id), int(tensor_id), int(sub_id)])


def normal_f32(shape, config_id, tensor_id, sub_id=0, std=1.0):
    """float32 draws from N(0, std^2)."""
    r = host_rng(config_id, tensor_id, sub_id)
    a = r.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    NaN is kept quiet."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def zipf_group_sizes(total_rows, num_groups, s, config_id, tensor_id,
                     forced_tail=(1, 0)):
    """Group sizes whose rank r has probability proportional to r^-s.

    Rows are dealt by a multinomial draw; the lowest-ranked groups are then
    forced to the sizes in ``forced_tail`` (so a 0-row and a 1-row group
    exist), the difference going to rank 1; finally ranks are mapped to
    group ids by a seeded permutation.  Returns int64 sizes [num_groups]."""
    r = host_rng(config_id, tensor_id, 0)
    ranks = np.arange(1, num_groups + 1, dtype=np.float64)
    p = ranks ** (-float(s))
    p /= p.sum()
    counts = r.multinomial(total_rows, p).astype(np.int64)
    for j, size in enumerate(forced_tail):
        idx = num_groups - 1 - j
        if idx <= 0:
            break
        diff = counts[idx] - size
        counts[idx] = size
        counts[0] += diff
    perm = host_rng(config_id, tensor_id, 1).permutation(num_groups)
    sizes = np.zeros(num_groups, dtype=np.int64)
    sizes[perm] = counts
    assert sizes.sum() == total_rows
    return sizes


def symmetric_int8_rows(a):
    """Input preparation for the int8 grouped GEMM: every row of ``a`` (last
    axis) is mapped to int8 with its own scale max|row|/127, values rounded
    half-to-even and clamped to [-127, 127].  A zero row gets scale 1.
    Returns (int8 array, float32 scales)."""
    a = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a), axis=-1, keepdims=True).astype(np.float32)
    scale = amax / np.float32(127.0)
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.clip(np.rint(a / scale), -127, 127).astype(np.int8)
    return q, scale[..., 0]


def device_normal_bf16(shape, seed, std, device):
    """bfloat16 tensor of N(0, std^2) drawn on ``device`` with a seeded
    torch generator (Philox on GPU); used for weights too large to draw on
    the host.  The float32 draw is rounded to bfloat16 by torch (RNE)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat_t = out.view(-1)
    n = flat_t.numel()
    slab = 1 << 28  # draw in slabs to bound the float32 temporary
    for start in range(0, n, slab):
        m = min(slab, n - start)
        tmp = torch.randn(m, generator=g, dtype=torch.float32, device=device)
        tmp.mul_(std)
        flat_t[start:start + m].copy_(tmp)
    return out


def device_normal_f32(shape, seed, std, device):
    """float32 tensor of N(0, std^2) drawn on ``device`` with a seeded torch
    generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    out.mul_(std)
    return out
