"""Benchmark of the fused-MoE forward path on one MI355X.

A step is one moe_forward of the prefill-shaped layer (T=4096, H=2048,
I=768, E=128, top-8 softmax with renormalisation): routing, alignment, the
gate_up GEMM with SiLU*up, the down GEMM with the routing weight, and the
top-k reduce, on seeded synthetic inputs already resident in HBM.  The
expert weights are in the packed tile layout (moe_pack_weights, done once
before timing, as at model load; its time is reported).  The headline value
is that step's throughput in TFLOP/s (6*T*topk*H*I algorithmic FLOPs,
padding excluded).  The same run measures the layer on plain [E, N, K]
weights, the decode-shaped layers (HBM GB/s over the touched experts'
weights), the int8 grouped GEMM, the routing workload and the tiny layer,
and times the oracle on a bounded sample of the prefill workload on the
host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
       python bench.py --component decode16|decode64|int8gmm|routing|tiny|w8a8
The second form runs one of the secondary measurements alone and prints its
result as one JSON object (for profiling a single workload).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (published)
PEAK_INT8_TOPS = 5033.2        # MI355X dense int8 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)

# HBM bytes per launch of the gate_up GEMM (the layer's dominant kernel, expert-wide tiles at
# block 32), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a 1 GiB copy: 457,972 KiB
# of FETCH_SIZE (x 2: 915,944 KiB read) + 49,152 KiB written
# (profiles/prefill_layer_wide_tiles.md).  Only valid for that kernel configuration; None for
# any other block size or once the kernel has changed since the counters were taken.
GATE_UP_TRAFFIC = {"block_m": 32, "bytes": 988258763}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def bf16_from_host(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class Timer:
    """HIP-event timing on torch's current stream (the binding's stream)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps):
        t = self.torch
        start = [t.cuda.Event(enable_timing=True) for _ in range(reps)]
        end = [t.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            start[i].record()
            fn()
            end[i].record()
        t.cuda.synchronize()
        ms = [s.elapsed_time(e) for s, e in zip(start, end)]
        return float(np.mean(ms)), float(np.median(ms))


FLUSH_BYTES = 1 << 30          # two halves, each larger than the 256 MB Infinity Cache


def flushed_events(torch, fn, reps, flush):
    """Mean and median of fn, each call event-timed after a write of the
    first half of the flush buffer and a read of its second half (outside the
    timed region), so no call finds the previous call's data in the Infinity
    Cache or an L2.  The read evicts the write's dirty lines as well: left in
    the Infinity Cache they would be written back during the timed call,
    about 20 us of HBM time that belongs to the flush."""
    start = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    end = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    half = flush.numel() // 2
    wr, rd = flush[:half], flush[half:].view(torch.int64)
    for i in range(reps):
        wr.fill_(i & 0x7f)
        rd.sum()
        start[i].record()
        fn()
        end[i].record()
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(start, end)]
    return dict(mean_ms=float(np.mean(ms)), median_ms=float(np.median(ms)), reps=reps)


def calibrate(torch, dev, timer):
    """Ceilings measured on this GPU, for context: hipBLASLt bf16 GEMMs (a
    dense 8192^3 and the prefill gate_up as one batched GEMM of 128 experts x
    256 tokens x 1536 x 2048) and a 1 GiB device copy.  Run right before the
    timed layer's warm-up, they also bring the GPU clock up."""
    res = {}
    a = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    c = torch.empty((8192, 8192), device=dev, dtype=torch.bfloat16)
    for _ in range(20):
        torch.matmul(a, b, out=c)
    mean, med = timer.run(lambda: torch.matmul(a, b, out=c), 50)
    res["hipblaslt_dense_8192"] = dict(ms=med, tflops=2.0 * 8192 ** 3 / med * 1e-9)
    del a, b, c
    xa = torch.randn((128, 256, 2048), device=dev, dtype=torch.bfloat16)
    wb = torch.randn((128, 2048, 1536), device=dev, dtype=torch.bfloat16)
    cb = torch.empty((128, 256, 1536), device=dev, dtype=torch.bfloat16)
    for _ in range(20):
        torch.bmm(xa, wb, out=cb)
    mean, med = timer.run(lambda: torch.bmm(xa, wb, out=cb), 50)
    res["hipblaslt_batched_gate_up"] = dict(ms=med, tflops=2.0 * 128 * 256 * 2048 * 1536 / med * 1e-9)
    del xa, wb, cb
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    mean, med = timer.run(lambda: dst.copy_(src), 20)
    res["device_copy_1gib"] = dict(ms=med, gbs=2.0 * (1 << 30) / med * 1e-6)
    del src, dst
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def wall_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def graph_of(torch, fn):
    """fn (after one eager call) captured in a HIP graph, for replay."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def layer_inputs(torch, cfg, dev):
    import synth
    sub = cfg.extra.get("sub", 0)
    x = synth.normal_f32((cfg.T, cfg.H), cfg.cid, 0, sub)
    g = synth.normal_f32((cfg.T, cfg.E), cfg.cid, 1, sub)
    x_dev = (torch.from_numpy(x).to(dev) if cfg.x_dtype == "f32"
             else bf16_from_host(torch, synth.f32_to_bf16_bits(x), dev))
    w1 = synth.device_normal_bf16((cfg.E, 2 * cfg.I, cfg.H), cfg.cid * 1000 + 2, cfg.w_std, dev)
    w2 = synth.device_normal_bf16((cfg.E, cfg.H, cfg.I), cfg.cid * 1000 + 3, cfg.w_std, dev)
    return x_dev, torch.from_numpy(g).to(dev), w1, w2, x, g


def pack(torch, moe, w1, w2, timer):
    """Packed copies of the layer's weights and the time the packing took."""
    p1 = moe.moe_pack_weights(w1, "silu_mul")
    p2 = moe.moe_pack_weights(w2, "none")
    ms, _ = timer.run(lambda: (moe.moe_pack_weights(w1, "silu_mul", packed=p1.data),
                               moe.moe_pack_weights(w2, "none", packed=p2.data)), 3)
    return p1, p2, ms


def device_quantize(torch, w):
    """Per-output-channel symmetric int8 of a device bf16 [E, N, K] tensor
    (input preparation for the int8 layer), one expert at a time."""
    E, N, K = w.shape
    q = torch.empty((E, N, K), dtype=torch.int8, device=w.device)
    s = torch.empty((E, N), dtype=torch.float32, device=w.device)
    for e in range(E):
        we = w[e].float()
        amax = we.abs().amax(dim=1, keepdim=True)
        se = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
        q[e] = torch.clamp(torch.round(we / se), -127, 127).to(torch.int8)
        s[e] = se.squeeze(1)
    return q, s


def w8a8_weights(torch, moe, w1, w2):
    """Packed int8 weights and their per-channel scales."""
    w1q, s1 = device_quantize(torch, w1)
    w2q, s2 = device_quantize(torch, w2)
    p1, p2 = moe.moe_pack_weights(w1q, "silu_mul"), moe.moe_pack_weights(w2q, "none")
    del w1q, w2q
    return p1, s1, p2, s2


def bench_w8a8(torch, moe, dev, steps, warmup, inputs=None):
    """The prefill layer with int8 weights and int8 activations
    (moe_forward_w8a8), on the prefill layer's inputs (made here if not
    given: x, gating, w1, w2 on the device)."""
    import synth
    cfg = synth.CONFIGS["prefill"]
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk
    if inputs is None:
        inputs = layer_inputs(torch, cfg, dev)[:4]
    x, g, w1, w2 = inputs
    q1, s1, q2, s2 = w8a8_weights(torch, moe, w1, w2)
    ws8 = torch.empty(moe.moe_forward_w8a8_workspace_size(T, H, I, E, K), dtype=torch.uint8,
                      device=dev)
    out = torch.empty_like(x)
    ms8 = wall_steps(torch, lambda: moe.moe_forward_w8a8(x, g, q1, s1, q2, s2, K, out=out,
                                                         workspace=ws8), steps, warmup)
    flops = 6.0 * T * K * H * I
    return dict(ms=ms8, tops=flops / ms8 * 1e-9, frac_int8=flops / ms8 * 1e-9 / PEAK_INT8_TOPS)


def bench_prefill(torch, moe, dev, steps, warmup, timer, plain=True, before=None):
    """The prefill layer.  before() runs right before the warm-up steps (the
    calibration GEMMs: GPU work that brings the clock up after the host-side
    set-up, so that a short timed region starts at the steady clock)."""
    import synth
    cfg = synth.CONFIGS["prefill"]
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk
    x, g, w1_plain, w2_plain, x_host, g_host = layer_inputs(torch, cfg, dev)
    w1, w2, pack_ms = pack(torch, moe, w1_plain, w2_plain, timer)
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def step():
        moe.moe_forward(x, g, w1, w2, K, out=out, workspace=ws)

    before_res = before() if before is not None else None
    ms = wall_steps(torch, step, steps, warmup)
    flops = 6.0 * T * K * H * I
    res = dict(ms=ms, tflops=flops / ms * 1e-9, flops=flops, pack_weights_ms=pack_ms,
               before=before_res)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    fl = flushed_events(torch, step, max(steps, 10), flush)
    fl["tflops"] = flops / fl["mean_ms"] * 1e-9
    res["flushed"] = fl

    def step_plain():
        moe.moe_forward(x, g, w1_plain, w2_plain, K, out=out, workspace=ws)

    if plain:
        ms_plain = wall_steps(torch, step_plain, steps, warmup)
        res["plain_weights"] = dict(ms=ms_plain, tflops=flops / ms_plain * 1e-9)
        # the same layer with int8 weights and int8 activations (moe_forward_w8a8)
        res["w8a8"] = bench_w8a8(torch, moe, dev, steps, warmup, (x, g, w1_plain, w2_plain))

    # Per-kernel breakdown: the launches moe_forward makes (route, the
    # two-kernel alignment, gate_up with SiLU*up, down with the routing
    # weight), each timed with HIP events on the stream they run on; the
    # top-k reduce is the rest of the step.  Inside moe_forward the
    # alignment also writes the expert-wide tile table; here the table comes
    # from moe_wide_tile_table (timed as tile_table, not part of the step).
    P = T * K
    bm = moe.moe_forward_block_m(T, E, K, "bf16", "packed")   # the block size used here
    w_t, ids_t = moe.moe_route(g, K)
    aws = torch.empty(moe.moe_align_workspace_size(P, E), dtype=torch.uint8, device=dev)
    sorted_ids, eids, total = moe.moe_align_block_size(ids_t, E, bm, workspace=aws)
    cap = sorted_ids.numel()
    h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((P, H), dtype=torch.bfloat16, device=dev)   # y in x's dtype
    torch.cuda.synchronize()
    reps = max(steps, 10)
    parts = {
        "route": lambda: moe.moe_route(g, K, topk_weights=w_t, topk_ids=ids_t),
        "align": lambda: moe.moe_align_block_size(ids_t, E, bm, sorted_ids, eids, total,
                                                  workspace=aws),
    }
    if bm == 32:   # expert-wide tiles, as moe_forward runs them for bf16 x
        table = moe.moe_wide_tile_table(eids, total, E, cap)
        parts["tile_table"] = lambda: moe.moe_wide_tile_table(eids, total, E, cap, table)
        parts["gemm1_gate_up_silu"] = lambda: moe.moe_grouped_gemm_wide(
            x, w1, sorted_ids, eids, total, table, P, a_rows="pair", a_row_div=K,
            epilogue="silu_mul", C=h, c_rows="sorted")
        parts["gemm2_down_weighted"] = lambda: moe.moe_grouped_gemm_wide(
            h, w2, sorted_ids, eids, total, table, P, a_rows="sorted", topk_weights=w_t,
            C=y, c_rows="pair")
    else:
        parts["gemm1_gate_up_silu"] = lambda: moe.moe_grouped_gemm(
            x, w1, sorted_ids, eids, total, bm, P, a_rows="pair", a_row_div=K,
            epilogue="silu_mul", C=h, c_rows="sorted")
        parts["gemm2_down_weighted"] = lambda: moe.moe_grouped_gemm(
            h, w2, sorted_ids, eids, total, bm, P, a_rows="sorted", topk_weights=w_t,
            C=y, c_rows="pair")
    br = {}
    for name, fn in parts.items():
        for _ in range(warmup):
            fn()
        mean, med = timer.run(fn, reps)
        br[name] = dict(mean_ms=mean, median_ms=med)
    br["gemm1_gate_up_silu"]["flushed"] = flushed_events(
        torch, parts["gemm1_gate_up_silu"], reps, flush)
    del flush
    gemm1_flops = 2.0 * P * H * 2 * I
    gemm2_flops = 2.0 * P * I * H
    br["gemm1_gate_up_silu"]["tflops"] = \
        gemm1_flops / br["gemm1_gate_up_silu"]["mean_ms"] * 1e-9
    br["gemm2_down_weighted"]["tflops"] = \
        gemm2_flops / br["gemm2_down_weighted"]["mean_ms"] * 1e-9
    # algorithmic HBM bytes of each GEMM launch: its weights, its token rows
    # read once, its output written once (bf16)
    gemm1_bytes = E * 2 * I * H * 2 + T * H * 2 + P * I * 2
    gemm2_bytes = E * H * I * 2 + P * I * 2 + P * H * 2
    for name, nb in (("gemm1_gate_up_silu", gemm1_bytes), ("gemm2_down_weighted", gemm2_bytes)):
        br[name]["algorithmic_bytes"] = nb
        br[name]["gbs"] = nb / br[name]["mean_ms"] * 1e-6
        br[name]["frac_hbm"] = br[name]["gbs"] / PEAK_HBM_GBS
    br["gemm1_gate_up_silu"]["flushed"]["gbs"] = \
        gemm1_bytes / br["gemm1_gate_up_silu"]["flushed"]["mean_ms"] * 1e-6
    br["remainder_reduce_and_gaps_ms"] = ms - sum(
        br[k]["mean_ms"] for k in parts if k != "tile_table")
    res["breakdown"] = br
    res["gemm1_flops"] = gemm1_flops
    res["gemm1_bytes"] = gemm1_bytes
    res["block_m"] = bm
    res["inputs"] = (x_host, g_host, w1_plain, w2_plain)
    return res


def touched_experts(ids):
    return int(np.unique(ids.reshape(-1)).size)


def bench_decode(torch, moe, dev, name, steps, warmup, timer):
    import synth
    cfg = synth.CONFIGS[name]
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk
    x, g, w1_plain, w2_plain, _, _ = layer_inputs(torch, cfg, dev)
    w1, w2, pack_ms = pack(torch, moe, w1_plain, w2_plain, timer)
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)

    def run(a, b):
        moe.moe_forward(x, g, a, b, K, cfg.groups, cfg.topk_group, "softmax", True, cfg.scale,
                        out=out, topk_ids_out=ids, workspace=ws)

    ms = wall_steps(torch, lambda: run(w1, w2), steps, warmup)
    n_exp = touched_experts(ids.cpu().numpy())
    per_expert = (2 * I * H + H * I) * 2
    nbytes = n_exp * per_expert + 2 * T * H * 2
    mean, med = timer.run(lambda: run(w1, w2), max(steps, 10))
    ms_plain = wall_steps(torch, lambda: run(w1_plain, w2_plain), steps, warmup)
    del w1, w2
    # int8 weights and activations: half the weight bytes
    q1, s1, q2, s2 = w8a8_weights(torch, moe, w1_plain, w2_plain)
    del w1_plain, w2_plain
    torch.cuda.empty_cache()
    ws8 = torch.empty(moe.moe_forward_w8a8_workspace_size(T, H, I, E, K), dtype=torch.uint8,
                      device=dev)

    def run8():
        moe.moe_forward_w8a8(x, g, q1, s1, q2, s2, K, cfg.groups, cfg.topk_group, "softmax", True,
                             cfg.scale, out=out, topk_ids_out=ids, workspace=ws8)

    ms8 = wall_steps(torch, run8, steps, warmup)
    nbytes8 = n_exp * (3 * I * H + 4 * (2 * I + H)) + 2 * T * H * 2
    del q1, q2, ws8
    torch.cuda.empty_cache()
    return dict(ms=ms, event_mean_ms=mean, touched_experts=n_exp, bytes=nbytes,
                gbs=nbytes / ms * 1e-6, frac_hbm=nbytes / ms * 1e-6 / PEAK_HBM_GBS,
                flops=6.0 * T * K * H * I, block_m=moe.moe_forward_block_m(T, E, K, "bf16", "packed"),
                pack_weights_ms=pack_ms,
                plain_weights=dict(ms=ms_plain, gbs=nbytes / ms_plain * 1e-6,
                                   block_m=moe.moe_forward_block_m(T, E, K)),
                w8a8=dict(ms=ms8, bytes=nbytes8, gbs=nbytes8 / ms8 * 1e-6,
                          frac_hbm=nbytes8 / ms8 * 1e-6 / PEAK_HBM_GBS))


def bench_int8(torch, moe, dev, steps, warmup, timer):
    import synth
    cfg = synth.CONFIGS["int8gmm"]
    M, K, N, E = cfg.T, cfg.H, cfg.I, cfg.E
    sizes = synth.zipf_group_sizes(M, E, cfg.extra["zipf_s"], cfg.cid, 9)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    xq, sx = synth.symmetric_int8_rows(synth.normal_f32((M, K), cfg.cid, 0))
    # weights: drawing 537M values on the host is slow; draw N(0, 0.02) on
    # the device and quantise per output channel there (input preparation).
    wf = synth.device_normal_f32((E, N, K), cfg.cid * 1000 + 1, cfg.w_std, dev)
    amax = wf.abs().amax(dim=2, keepdim=True)
    sw = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
    wq = torch.clamp(torch.round(wf / sw), -127, 127).to(torch.int8)
    sw = sw.squeeze(2).contiguous()
    del wf, amax
    xq_d = torch.from_numpy(xq).to(dev)
    sx_d = torch.from_numpy(sx).to(dev)
    off_d = torch.from_numpy(off).to(dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    wp = moe.moe_pack_weights(wq)           # packed once, as at model load

    def step():
        moe.gmm_int8(xq_d, wp, sx_d, sw, off_d, output=Y)

    ms = wall_steps(torch, step, steps, warmup)
    mean, med = timer.run(step, max(steps, 10))
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    fl = flushed_events(torch, step, max(steps, 10), flush)
    del flush
    ms_plain = wall_steps(torch, lambda: moe.gmm_int8(xq_d, wq, sx_d, sw, off_d, output=Y),
                          steps, warmup)
    nz = int((sizes > 0).sum())
    nbytes = nz * N * K + M * K + 2 * M * N + 4 * (E * N + M)
    ops = 2.0 * M * N * K
    del wq, wp
    torch.cuda.empty_cache()
    return dict(ms=ms, event_mean_ms=mean, tops=ops / ms * 1e-9, gbs=nbytes / ms * 1e-6,
                frac_hbm=nbytes / ms * 1e-6 / PEAK_HBM_GBS,
                frac_int8=ops / ms * 1e-9 / PEAK_INT8_TOPS, bytes=nbytes, ops=ops,
                weights="packed", plain_weights=dict(ms=ms_plain, gbs=nbytes / ms_plain * 1e-6),
                flushed=dict(fl, gbs=nbytes / fl["mean_ms"] * 1e-6,
                             frac_hbm=nbytes / fl["mean_ms"] * 1e-6 / PEAK_HBM_GBS),
                group_sizes_min_max=[int(sizes.min()), int(sizes.max())])


def bench_routing(torch, moe, dev, steps, warmup, timer):
    import synth
    cfg = synth.CONFIGS["routing"]
    g = torch.from_numpy(synth.normal_f32((cfg.T, cfg.E), cfg.cid, 0)).to(dev)
    w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=dev)
    ids = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=dev)

    def step():
        moe.moe_route(g, cfg.topk, cfg.groups, cfg.topk_group, "softmax", True, 1.0, w, ids)

    ms = wall_steps(torch, step, steps * 10, warmup)
    mean, med = timer.run(step, 100)
    return dict(ms_wall=ms, event_median_us=med * 1e3, event_mean_us=mean * 1e3,
                input_bytes=cfg.T * cfg.E * 4)


def bench_tiny(torch, moe, dev, steps, warmup, timer):
    import synth
    cfg = synth.CONFIGS["tiny"]
    x = torch.from_numpy(synth.normal_f32((cfg.T, cfg.H), cfg.cid, 0)).to(dev)
    g = torch.from_numpy(synth.normal_f32((cfg.T, cfg.E), cfg.cid, 1)).to(dev)
    w1 = bf16_from_host(torch, synth.f32_to_bf16_bits(
        synth.normal_f32((cfg.E, 2 * cfg.I, cfg.H), cfg.cid, 2, 0, cfg.w_std)), dev)
    w2 = bf16_from_host(torch, synth.f32_to_bf16_bits(
        synth.normal_f32((cfg.E, cfg.H, cfg.I), cfg.cid, 3, 0, cfg.w_std)), dev)
    ws = torch.empty(moe.moe_forward_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def step():
        moe.moe_forward(x, g, w1, w2, cfg.topk, out=out, workspace=ws)

    ms = wall_steps(torch, step, steps * 10, warmup)
    mean, med = timer.run(step, 100)
    # the same call captured once in a HIP graph and replayed (one graph
    # launch per layer instead of one launch per kernel)
    graph = graph_of(torch, step)
    ms_g = wall_steps(torch, graph.replay, steps * 10, warmup)
    _, med_g = timer.run(graph.replay, 100)
    return dict(ms_wall=ms, event_median_us=med * 1e3, graph_ms_wall=ms_g,
                graph_event_median_us=med_g * 1e3)


def cpu_baseline(torch, prefill_inputs, target_s=12.0):
    """The oracle, as it stands, on the first S tokens of the prefill batch
    (all of them, repeated, when one pass is shorter than the target).
    Weights are decoded from bf16 to float64 before the timed region."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    cfg = synth.CONFIGS["prefill"]
    x_host, g_host, w1, w2 = prefill_inputs
    xb = oracle.bf16_bits_to_f64(synth.f32_to_bf16_bits(x_host))
    w1h = oracle.bf16_bits_to_f64(w1.view(torch.int16).cpu().numpy().view(np.uint16))
    w2h = oracle.bf16_bits_to_f64(w2.view(torch.int16).cpu().numpy().view(np.uint16))
    g64 = g_host.astype(np.float64)
    def one(S):
        w, ids = oracle.grouped_topk(g64[:S], cfg.topk)
        oracle.moe_layer_expert_loop(xb[:S], w1h, w2h, w, ids)

    S = 64
    while True:
        t0 = time.perf_counter()
        one(S)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or S >= cfg.T:
            break
        S = min(cfg.T, int(S * min(8.0, max(2.0, target_s / max(dt, 1e-3)))))
    reps = max(1, int(round(target_s / max(dt, 1e-3)))) if S >= cfg.T else 1
    t0 = time.perf_counter()
    for _ in range(reps):
        one(S)
    dt = (time.perf_counter() - t0) / reps
    flops = 6.0 * S * cfg.topk * cfg.H * cfg.I
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return dict(value=flops / dt * 1e-12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(), seconds_per_pass=dt, passes=reps,
                sample="%d pass(es) over the first %d of %d tokens of the prefill layer (route + "
                       "expert-loop layer, float64 NumPy; weights pre-decoded)" % (reps, S, cfg.T))


def copy_calibration(torch, dev):
    """Three 1 GiB device-to-device copies: known HBM bytes for scaling the
    byte counters of a profiled run."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # enough warm-up for the GPU clock to settle after the host-side set-up
    # of each measurement (about 50 ms of kernels); the timed steps are short
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--quick", action="store_true", help="prefill headline only")
    ap.add_argument("--component", choices=["decode16", "decode64", "int8gmm", "routing", "tiny",
                                            "w8a8"],
                    help="run this secondary measurement alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain", action="store_true",
                    help="skip the plain-layout comparison runs (profiling the measured path only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also copy 1 GiB device-to-device 3 times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(collectives are out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_topk_amd as moe
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    timer = Timer(torch)

    if args.component:
        log(args.component)
        fn = {"decode16": lambda: bench_decode(torch, moe, dev, "decode16", args.steps, args.warmup,
                                               timer),
              "decode64": lambda: bench_decode(torch, moe, dev, "decode64", args.steps, args.warmup,
                                               timer),
              "int8gmm": lambda: bench_int8(torch, moe, dev, args.steps, args.warmup, timer),
              "routing": lambda: bench_routing(torch, moe, dev, args.steps, args.warmup, timer),
              "tiny": lambda: bench_tiny(torch, moe, dev, args.steps, args.warmup, timer),
              "w8a8": lambda: bench_w8a8(torch, moe, dev, args.steps, args.warmup)}
        res = fn[args.component]()
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({"component": args.component, "steps": args.steps,
                          "warmup": args.warmup, "result": res}), flush=True)
        return

    log("prefill layer (calibration GEMMs and copy right before its warm-up)")
    pre = bench_prefill(torch, moe, dev, args.steps, args.warmup, timer, plain=not args.no_plain,
                        before=lambda: calibrate(torch, dev, timer))
    calib = pre["before"]
    g1 = pre["breakdown"]["gemm1_gate_up_silu"]
    # MFMA is the graded bound; at this shape HBM co-binds (206 GFLOP over
    # 872 MB of weights, tokens and h: 236 FLOP/B, under the 315 FLOP/B
    # ridge), so the attainable fraction of the MFMA peak is 236 / 315
    ai = pre["gemm1_flops"] / pre["gemm1_bytes"]
    attainable = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS * 1e-3)
    roofline = dict(bound="mfma", achieved=g1["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=g1["tflops"] / PEAK_BF16_TFLOPS,
                    traffic=(GATE_UP_TRAFFIC["bytes"] if pre["block_m"] == GATE_UP_TRAFFIC["block_m"]
                             else None),
                    traffic_unit="bytes per launch",
                    kernel=("moe_gemm_wide_kernel<1>, gate_up with the SiLU*up epilogue on "
                            "expert-wide tiles (the layer's dominant kernel), packed weights"
                            if pre["block_m"] == 32 else
                            "moe_gemm_dma_kernel, gate_up with the SiLU*up epilogue (the layer's "
                            "dominant kernel), packed weights"),
                    block_m=pre["block_m"],
                    flops_per_launch=pre["gemm1_flops"], mean_ms=g1["mean_ms"],
                    hbm=dict(algorithmic_bytes=pre["gemm1_bytes"], achieved_gbs=g1["gbs"],
                             peak_gbs=PEAK_HBM_GBS, frac=g1["frac_hbm"],
                             flop_per_byte=ai, attainable_tflops=attainable,
                             frac_of_attainable=g1["tflops"] / attainable))
    components = {"calibration": calib, "prefill_flushed": pre["flushed"],
                  "prefill_breakdown": pre["breakdown"], "prefill_plain_weights": pre.get("plain_weights"),
                  "prefill_w8a8": pre.get("w8a8"), "prefill_pack_weights_ms": pre["pack_weights_ms"]}
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not args.quick:
        for name in ("decode16", "decode64"):
            log(name)
            components[name] = bench_decode(torch, moe, dev, name, args.steps, args.warmup, timer)
        log("int8 gmm")
        components["int8gmm"] = bench_int8(torch, moe, dev, args.steps, args.warmup, timer)
        log("routing")
        components["routing"] = bench_routing(torch, moe, dev, args.steps, args.warmup, timer)
        log("tiny")
        components["tiny"] = bench_tiny(torch, moe, dev, args.steps, args.warmup, timer)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(torch, pre["inputs"])

    line = {
        "metric": "fused-MoE layer TFLOP/s + decode HBM GB/s at 1 GPU, as % of MI355X roofline",
        "value": round(pre["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill-shaped MoE layer forward", "T": 4096, "H": 2048,
                   "I": 768, "E": 128, "topk": 8, "routing": "softmax top-8, renormalize",
                   "frac_of_bf16_peak": round(pre["tflops"] / PEAK_BF16_TFLOPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": components,
    }
    if "decode16" in components:
        line["decode_gbs"] = {k: round(components[k]["gbs"], 1) for k in ("decode16", "decode64")}
        line["decode_frac_hbm"] = {k: round(components[k]["frac_hbm"], 4)
                                   for k in ("decode16", "decode64")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
