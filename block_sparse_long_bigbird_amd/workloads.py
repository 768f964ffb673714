"""Seeded synthetic workloads for BigBird block-sparse attention.

This module only draws inputs: shapes, value distributions and padding
patterns.  It holds none of the attention arithmetic, so the HIP path and the
fp64 oracle can both be fed from it without sharing any of the method.

Shapes stand in for the workloads the pages describe: BigBird-base and
BigBird-large pretraining at 4096 tokens (12 heads x 64 and 16 heads x 64,
block 64, 3 random blocks; page "Big Bird: Transformers for Longer Sequences",
section "计算设置", and page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
encoder parameter table), 16K-token Path-X-length inputs, and 32K-token
documents (paper card, section "瓶颈", for the document-length statistics).
No dataset is used: every value is a seeded draw.

Recipe (per workload): numpy Generator(PCG64(data_seed)); draw q, then k, then
v as float32 N(0,1) of shape [B, H, L, d]; then the padding lengths; then the
key outlier rows.  Values are multiplied by `value_scale`, outlier key rows by
`outlier_mult`, and the result is rounded once to the compute dtype (bf16:
round-to-nearest-even via torch).  The rounded tensor is what both the GPU and
the oracle see.  The random-block table is built from `rand_seed` by the
library's adjacency builder, not here.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    block: int
    r: int
    dtype: str                 # "fp32" or "bf16"
    value_scale: float         # N(0,1) draws are multiplied by this
    pad: str                   # "none" | "per_seq_blocks" | "fixed" | "scattered"
    valid_len: int = 0         # for pad == "fixed"
    pad_lo_blocks: int = 0     # for pad == "per_seq_blocks": valid = block*U{lo..hi}
    pad_hi_blocks: int = 0
    outlier_frac: float = 0.0  # fraction of key rows per (b, h) scaled by outlier_mult
    outlier_mult: float = 1.0
    data_seed: int = 0
    rand_seed: int = 0         # seed of the random-block table (layer index 0)

    @property
    def nb(self) -> int:
        return self.L // self.block

    @property
    def tokens(self) -> int:
        return self.B * self.L


WORKLOADS = {
    # fp32, tiny: the case the oracle finishes in seconds.
    "fp32_B1_H2_L1024": Workload(
        "fp32_B1_H2_L1024", B=1, H=2, L=1024, d=64, block=64, r=3, dtype="fp32",
        value_scale=1.0, pad="none", data_seed=1),
    # BigBird-base attention layer shape with per-sequence padding.
    "base_B4_H12_L4096_pad": Workload(
        "base_B4_H12_L4096_pad", B=4, H=12, L=4096, d=64, block=64, r=3, dtype="bf16",
        value_scale=1.0 / 8.0, pad="per_seq_blocks", pad_lo_blocks=32, pad_hi_blocks=64,
        data_seed=2),
    # BigBird-large attention shape.
    "large_B8_H16_L4096": Workload(
        "large_B8_H16_L4096", B=8, H=16, L=4096, d=64, block=64, r=3, dtype="bf16",
        value_scale=1.0 / 8.0, pad="none", data_seed=3),
    # 16K tokens (Path-X length), last 1024 tokens padded.
    "pathx_B1_H8_L16384_pad": Workload(
        "pathx_B1_H8_L16384_pad", B=1, H=8, L=16384, d=64, block=64, r=3, dtype="bf16",
        value_scale=1.0 / 8.0, pad="fixed", valid_len=15360, data_seed=4),
    # 32K tokens, block 128, 4 random blocks, 1% of key rows x8.
    "long_B1_H12_L32768_bs128": Workload(
        "long_B1_H12_L32768_bs128", B=1, H=12, L=32768, d=64, block=128, r=4, dtype="bf16",
        value_scale=1.0 / 8.0, pad="none", outlier_frac=0.01, outlier_mult=8.0, data_seed=5),
}

# Order of the workloads as the performance table lists them.
WORKLOAD_ORDER = list(WORKLOADS)

# Supplementary softmax stress case (not a benchmark line): the 32K shape with
# unscaled N(0,1) values, so the x8 key outliers move the running row maximum.
STRESS_LONG = replace(WORKLOADS["long_B1_H12_L32768_bs128"],
                      name="stress_long_unscaled", value_scale=1.0, data_seed=6)


def draw(w: Workload):
    """Seeded float32 draws (before rounding to the compute dtype).

    Returns (q, k, v, pad) with q/k/v float32 [B, H, L, d] and pad a uint8
    [B, L] array (1 = valid token, 0 = padding) or None.
    """
    rng = np.random.Generator(np.random.PCG64(w.data_seed))
    shape = (w.B, w.H, w.L, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.value_scale != 1.0:
        s = np.float32(w.value_scale)
        q *= s
        k *= s
        v *= s
    pad = None
    if w.pad == "per_seq_blocks":
        nblk = rng.integers(w.pad_lo_blocks, w.pad_hi_blocks + 1, size=w.B)
        valid = nblk * w.block
        pad = (np.arange(w.L)[None, :] < valid[:, None]).astype(np.uint8)
    elif w.pad == "fixed":
        pad = np.zeros((w.B, w.L), dtype=np.uint8)
        pad[:, : w.valid_len] = 1
    elif w.pad == "scattered":
        # holes anywhere, from their own stream (PCG64 seeded with data_seed + 3000):
        # each token padded with probability 0.3, plus one padded span of 1.5 blocks
        # per sequence (whole padded 32-key subtiles between valid ones)
        prng = np.random.Generator(np.random.PCG64(w.data_seed + 3000))
        pad = (prng.random((w.B, w.L)) >= 0.3).astype(np.uint8)
        span = 3 * w.block // 2
        for b in range(w.B):
            s0 = int(prng.integers(0, w.L - span + 1))
            pad[b, s0:s0 + span] = 0
    elif w.pad != "none":
        raise ValueError(f"unknown pad mode {w.pad!r}")
    if w.outlier_frac > 0.0:
        n_out = int(np.floor(w.outlier_frac * w.L))
        m = np.float32(w.outlier_mult)
        for b in range(w.B):
            for h in range(w.H):
                rows = rng.choice(w.L, size=n_out, replace=False)
                k[b, h, rows, :] *= m
    return q, k, v, pad


def torch_dtype(name: str):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload):
    """Inputs rounded to the compute dtype, as CPU torch tensors.

    Returns (q, k, v, pad) -- q/k/v in the workload's dtype, pad a uint8
    tensor [B, L] or None.
    """
    import torch
    q, k, v, pad = draw(w)
    dt = torch_dtype(w.dtype)
    tq = torch.from_numpy(q).to(dt)
    tk = torch.from_numpy(k).to(dt)
    tv = torch.from_numpy(v).to(dt)
    tpad = None if pad is None else torch.from_numpy(pad)
    return tq, tk, tv, tpad


def make_inputs_device(w: Workload, dev):
    """q, k, v drawn on the device, for shapes too large to draw on the host:
    N(0, 1) from torch's device generator seeded with data_seed (q, then k,
    then v), times value_scale, rounded to the compute dtype.  No padding, no
    outliers.  Returns (q, k, v) device tensors [B, H, L, d]."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(w.data_seed)
    out = []
    for _ in range(3):
        t = torch.randn((w.B, w.H, w.L, w.d), generator=g, device=dev, dtype=torch.float32)
        t.mul_(w.value_scale)
        out.append(t.to(torch_dtype(w.dtype)))
        del t
    return tuple(out)


def make_dout_device(w: Workload, dev):
    """Upstream gradient drawn on the device for the shapes of make_inputs_device:
    N(0, 1) from torch's device generator seeded with data_seed + 1000, rounded
    to the compute dtype.  Returns a device tensor [B, H, L, d]."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(w.data_seed + 1000)
    t = torch.randn((w.B, w.H, w.L, w.d), generator=g, device=dev, dtype=torch.float32)
    return t.to(torch_dtype(w.dtype))


def small(name: str, B: int, H: int, L: int, block: int, r: int, dtype: str = "bf16",
          d: int = 64, value_scale: float = 1.0, pad: str = "none", valid_len: int = 0,
          pad_lo_blocks: int = 0, pad_hi_blocks: int = 0, outlier_frac: float = 0.0,
          outlier_mult: float = 1.0, data_seed: int = 100, rand_seed: int = 0) -> Workload:
    """A small ad-hoc workload for parity tests."""
    return Workload(name, B=B, H=H, L=L, d=d, block=block, r=r, dtype=dtype,
                    value_scale=value_scale, pad=pad, valid_len=valid_len,
                    pad_lo_blocks=pad_lo_blocks, pad_hi_blocks=pad_hi_blocks,
                    outlier_frac=outlier_frac, outlier_mult=outlier_mult,
                    data_seed=data_seed, rand_seed=rand_seed)


def make_dout(w: Workload):
    """Upstream gradient for a backward pass: N(0,1) draws of shape [B, H, L, d]
    from its own stream (PCG64 seeded with data_seed + 1000), rounded to the
    workload's dtype, as a CPU torch tensor."""
    import torch
    rng = np.random.Generator(np.random.PCG64(w.data_seed + 1000))
    g = rng.standard_normal((w.B, w.H, w.L, w.d), dtype=np.float32)
    return torch.from_numpy(g).to(torch_dtype(w.dtype))


def make_layer_inputs(w: Workload):
    """Hidden states and synthetic projection weights for the attention layer of
    a workload's shape (hidden = H * d), as CPU torch tensors from their own
    stream (PCG64 seeded with data_seed + 2000): x ~ N(0, 1) [B, L, hidden] and
    the weights ~ N(0, 1/hidden) [out, in], both rounded to bf16; biases
    ~ N(0, 0.02^2) in float32; plus the workload's pad mask (or None)."""
    import torch
    hid = w.H * w.d
    rng = np.random.Generator(np.random.PCG64(w.data_seed + 2000))
    x = rng.standard_normal((w.B, w.L, hid), dtype=np.float32)
    s = np.float32(1.0 / np.sqrt(hid))
    w_qkv = rng.standard_normal((3 * hid, hid), dtype=np.float32) * s
    b_qkv = rng.standard_normal(3 * hid, dtype=np.float32) * np.float32(0.02)
    w_o = rng.standard_normal((hid, hid), dtype=np.float32) * s
    b_o = rng.standard_normal(hid, dtype=np.float32) * np.float32(0.02)
    _, _, _, pad = draw(w)
    bf = torch.bfloat16
    return (torch.from_numpy(x).to(bf), torch.from_numpy(w_qkv).to(bf), torch.from_numpy(b_qkv),
            torch.from_numpy(w_o).to(bf), torch.from_numpy(b_o),
            None if pad is None else torch.from_numpy(pad))


def make_stack_weights(w: Workload, n_layers: int):
    """Per-layer projection weights for a stack of n_layers attention layers of
    a workload's shape: layer l draws (w_qkv, b_qkv, w_o, b_o) as
    make_layer_inputs does, from its own stream (PCG64 seeded with
    data_seed + 3000 + l).  CPU torch tensors, weights bf16, biases float32."""
    import torch
    hid = w.H * w.d
    s = np.float32(1.0 / np.sqrt(hid))
    out = []
    for l in range(n_layers):
        rng = np.random.Generator(np.random.PCG64(w.data_seed + 3000 + l))
        w_qkv = rng.standard_normal((3 * hid, hid), dtype=np.float32) * s
        b_qkv = rng.standard_normal(3 * hid, dtype=np.float32) * np.float32(0.02)
        w_o = rng.standard_normal((hid, hid), dtype=np.float32) * s
        b_o = rng.standard_normal(hid, dtype=np.float32) * np.float32(0.02)
        out.append((torch.from_numpy(w_qkv).to(torch.bfloat16), torch.from_numpy(b_qkv),
                    torch.from_numpy(w_o).to(torch.bfloat16), torch.from_numpy(b_o)))
    return out
