"""Helpers of the GPU tests: moving seeded inputs to the device and exact
copies of device tensors back to the host for the oracle."""

import numpy as np
import torch

import oracle
import synth


def require_gpu():
    assert torch.cuda.is_available(), "the gpu-marked tests need a ROCm device"
    return torch.device("cuda:0")


def bf16_dev(bits, dev):
    """uint16 bfloat16 bit patterns (numpy) -> device bfloat16 tensor."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_host_f64(t):
    """Device/host bfloat16 tensor -> float64 numpy array (exact)."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(bits)


class LazyExperts:
    """Indexable stand-in for a huge [E, ...] bfloat16 device tensor: the
    oracle asks for one expert at a time and gets its exact float64 values."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return bf16_host_f64(self.t[int(e)])

    def __len__(self):
        return self.shape[0]


def layer_inputs(cfg, dev, x_dtype=None):
    """x, gating and expert weights of a fused-MoE layer config.
    Small weights are drawn on the host (PCG64); large ones on the device."""
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    sub = cfg.extra.get("sub", 0)
    x_dtype = x_dtype or cfg.x_dtype
    xf = synth.normal_f32((T, H), cfg.cid, 0, sub)
    gating = synth.normal_f32((T, E), cfg.cid, 1, sub)
    if x_dtype == "f32":
        x_dev = torch.from_numpy(xf).to(dev)
        x_host = xf.astype(np.float64)
    else:
        bits = synth.f32_to_bf16_bits(xf)
        x_dev = bf16_dev(bits, dev)
        x_host = oracle.bf16_bits_to_f64(bits)
    nbytes = 2 * E * 3 * I * H
    if nbytes <= (256 << 20):
        w1b = synth.f32_to_bf16_bits(synth.normal_f32((E, 2 * I, H), cfg.cid, 2, 0, cfg.w_std))
        w2b = synth.f32_to_bf16_bits(synth.normal_f32((E, H, I), cfg.cid, 3, 0, cfg.w_std))
        w1 = bf16_dev(w1b, dev)
        w2 = bf16_dev(w2b, dev)
        w1_host = oracle.bf16_bits_to_f64(w1b)
        w2_host = oracle.bf16_bits_to_f64(w2b)
    else:
        w1 = synth.device_normal_bf16((E, 2 * I, H), cfg.cid * 1000 + 2, cfg.w_std, dev)
        w2 = synth.device_normal_bf16((E, H, I), cfg.cid * 1000 + 3, cfg.w_std, dev)
        w1_host = LazyExperts(w1)
        w2_host = LazyExperts(w2)
    return dict(x=x_dev, x_host=x_host, gating=torch.from_numpy(gating).to(dev),
                gating_host=gating.astype(np.float64), w1=w1, w2=w2, w1_host=w1_host,
                w2_host=w2_host)


def gmm_inputs(M, K, N, E, sizes, seed, dev, w_std=0.02):
    """Expert-sorted int8 GMM inputs: per-token int8 activations and
    per-channel int8 weights with their scales (input preparation)."""
    sizes = np.asarray(sizes, dtype=np.int64)
    assert sizes.sum() == M
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    x = synth.normal_f32((M, K), seed, 0)
    xq, sx = synth.symmetric_int8_rows(x)
    wq = np.empty((E, N, K), dtype=np.int8)
    sw = np.empty((E, N), dtype=np.float32)
    w_f32 = {}
    for e in range(E):
        w = synth.normal_f32((N, K), seed, 1, e, w_std)
        wq[e], sw[e] = synth.symmetric_int8_rows(w)
        if E * N * K <= (1 << 24):
            w_f32[e] = w
    host = dict(xq=xq, sx=sx, wq=wq, sw=sw, off=off, x=x, w_f32=w_f32)
    devd = dict(xq=torch.from_numpy(xq).to(dev), sx=torch.from_numpy(sx).to(dev),
                wq=torch.from_numpy(wq).to(dev), sw=torch.from_numpy(sw).to(dev),
                off=torch.from_numpy(off).to(dev))
    return host, devd
