"""GPU parity of the attention layer (bb_layer_forward) against the fp64
oracle's layer_forward.

Tolerance: max |gpu - oracle| <= 2e-2 * max |oracle| per case.  The layer
keeps q, k, v and the attention output in bf16 between its steps (relative
rounding 2^-9 each, fp32 accumulation inside every product) and rounds y to
bf16.  The output is NaN-poisoned first and scanned.
"""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import WORKLOADS, make_layer_inputs, small
from oracle import layer_forward, layer_rows

pytestmark = pytest.mark.gpu
REL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()
    return torch.device("cuda:0")


def run_layer(w, dev, inputs, ri):
    x, w_qkv, b_qkv, w_o, b_o, pad = inputs
    hid = w.H * w.d
    y = torch.full((w.B, w.L, hid), float("nan"), dtype=torch.bfloat16, device=dev)
    n = bb.bb_layer_workspace_bytes(w.B, w.L, hid, w.H, w.block)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    say(f"  layer {w.name} B={w.B} L={w.L} hidden={hid} H={w.H} block={w.block} r={w.r}")
    bb.bb_layer_forward(x.to(dev), w_qkv.to(dev), b_qkv.to(dev), w_o.to(dev), b_o.to(dev),
                        None if pad is None else pad.to(dev),
                        torch.from_numpy(ri).to(dev) if w.r > 0 else None,
                        w.B, w.L, hid, w.H, w.block, w.r, y, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def f64(t):
    return t.to(torch.float64).numpy()


def check(w, dev):
    inputs = make_layer_inputs(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_layer(w, dev, inputs, ri)
    x, w_qkv, b_qkv, w_o, b_o, pad = inputs
    exp = layer_forward(f64(x), f64(w_qkv), b_qkv.numpy().astype(np.float64), f64(w_o),
                        b_o.numpy().astype(np.float64), None if pad is None else pad.numpy(), ri, w.H,
                        w.block)
    assert not np.isnan(got).any(), "unwritten (NaN) outputs"
    err, scale = np.abs(got - exp).max(), np.abs(exp).max()
    say(f"  max err {err:.3e}  max |ref| {scale:.3e}  rel {err / scale:.3e}")
    assert err <= REL * scale


LAYER_CASES = [
    small("layer_h128_nb4", B=1, H=2, L=4 * 64, block=64, r=0, data_seed=71),
    small("layer_h256_nb8_r3_pad", B=2, H=4, L=8 * 64, block=64, r=3, pad="fixed",
          valid_len=8 * 64 - 77, data_seed=72),
    small("layer_h128_bs128_nb6_r1", B=1, H=2, L=6 * 128, block=128, r=1, data_seed=73),
    small("layer_h768_nb10_r3", B=1, H=12, L=10 * 64 + 128, block=64, r=3, data_seed=74),
    # B*L a multiple of 256 but L not: the QKV projection's 256-row tiles
    # straddle the two sequences; the output projection takes 128-row tiles
    small("layer_h768_B2_L384_pad", B=2, H=12, L=6 * 64, block=64, r=1, pad="fixed",
          valid_len=6 * 64 - 50, data_seed=75),
]


@pytest.mark.parametrize("w", LAYER_CASES, ids=[w.name for w in LAYER_CASES])
def test_layer_matches_oracle(dev, w):
    check(w, dev)


def test_layer_full_size_one_sequence(dev):
    """BigBird-base shape (hidden 768, 12 heads, L 4096, padded) for one sequence."""
    base = WORKLOADS["base_B4_H12_L4096_pad"]
    w = small("layer_base_B1", B=1, H=base.H, L=base.L, block=base.block, r=base.r,
              pad="fixed", valid_len=base.L - 1000, value_scale=base.value_scale, data_seed=75)
    check(w, dev)


def test_layer_full_size_bench_configuration_sampled(dev):
    """The benchmark's layer configuration exactly (BigBird-base shape, B 4, L 4096,
    hidden 768, 12 heads, per-sequence padding, the benchmark's inputs and
    table): sampled output rows of every sequence against the oracle's
    layer_rows (global blocks, block edges, padded rows, random picks)."""
    w = WORKLOADS["base_B4_H12_L4096_pad"]
    inputs = make_layer_inputs(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_layer(w, dev, inputs, ri)
    assert not np.isnan(got).any(), "unwritten (NaN) outputs"
    rng = np.random.default_rng(76)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 65, 127, 2047, 2048, 2049, 4031, 4032, 4095],
                                     rng.integers(0, w.L, 8)]))
    x, w_qkv, b_qkv, w_o, b_o, pad = inputs
    exp = layer_rows(f64(x), f64(w_qkv), b_qkv.numpy().astype(np.float64), f64(w_o),
                     b_o.numpy().astype(np.float64), None if pad is None else pad.numpy(), ri, w.H,
                     w.block, rows)
    err, scale = np.abs(got[:, rows] - exp).max(), np.abs(exp).max()
    say(f"  {len(rows)} rows x {w.B} sequences: max err {err:.3e}  max |ref| {scale:.3e}  rel {err / scale:.3e}")
    assert err <= REL * scale


def run_stack(w, dev, x, layers, pad, tables):
    hid = w.H * w.d
    y = torch.full((w.B, w.L, hid), float("nan"), dtype=torch.bfloat16, device=dev)
    n = bb.bb_layer_stack_workspace_bytes(w.B, w.L, hid, w.H, w.block)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    dl = [tuple(t.to(dev) for t in lw) + (torch.from_numpy(ri).to(dev) if w.r > 0 else None,)
          for lw, ri in zip(layers, tables)]
    say(f"  stack {w.name} layers={len(layers)} B={w.B} L={w.L} hidden={hid} H={w.H} block={w.block} r={w.r}")
    bb.bb_layer_stack_forward(x.to(dev), dl, None if pad is None else pad.to(dev), w.B, w.L, hid, w.H,
                              w.block, w.r, y, ws)
    torch.cuda.synchronize()
    return y


STACK_CASES = [
    (3, small("stack_h256_nb8_r3_pad", B=2, H=4, L=8 * 64, block=64, r=3, pad="fixed",
              valid_len=8 * 64 - 77, data_seed=81)),
    (4, small("stack_h128_bs128_nb6_r1", B=1, H=2, L=6 * 128, block=128, r=1, data_seed=82)),
]


@pytest.mark.parametrize("n_layers,w", STACK_CASES, ids=[f"{w.name}_x{n}" for n, w in STACK_CASES])
def test_layer_stack_per_layer_tables(dev, n_layers, w):
    """A stack of layers, layer l with its own weights and the table seeded
    with l: (1) bit-identical to the layers called one after another with
    bb_layer_forward; (2) its last layer against the oracle's layer applied to
    the output of the stack one layer shorter; (3) the whole stack against the
    oracle's stack in fp64 (errors add up over the layers); (4) the tables of
    different layers differ."""
    from block_sparse_long_bigbird_amd.workloads import make_stack_weights
    from oracle import layer_stack_forward

    x, _, _, _, _, pad = make_layer_inputs(w)
    layers = make_stack_weights(w, n_layers)
    tables = [bb.bb_rand_idx_build(l, w.H, w.L, w.block, w.r) for l in range(n_layers)]
    if w.r > 0:
        assert not np.array_equal(tables[0], tables[1])
    y = run_stack(w, dev, x, layers, pad, tables)
    assert not torch.isnan(y.float()).any(), "unwritten (NaN) outputs"
    # (1) one call per layer
    hid = w.H * w.d
    cur = x.to(dev)
    for l, (lw, ri) in enumerate(zip(layers, tables)):
        nxt = torch.empty_like(cur)
        n = bb.bb_layer_workspace_bytes(w.B, w.L, hid, w.H, w.block)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        bb.bb_layer_forward(cur, *(t.to(dev) for t in lw), None if pad is None else pad.to(dev),
                            torch.from_numpy(ri).to(dev) if w.r > 0 else None,
                            w.B, w.L, hid, w.H, w.block, w.r, nxt, ws)
        if l == n_layers - 2:
            before_last = nxt
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(y, cur), "stack differs from one call per layer"
    # (2) the last layer from the GPU's input to it
    lw, ri = layers[-1], tables[-1]
    pd = None if pad is None else pad.numpy()
    exp = layer_forward(f64(before_last.cpu()), f64(lw[0]), lw[1].numpy().astype(np.float64), f64(lw[2]),
                        lw[3].numpy().astype(np.float64), pd, ri, w.H, w.block)
    got = y.float().cpu().numpy()
    err, scale = np.abs(got - exp).max(), np.abs(exp).max()
    say(f"  last layer: max err {err:.3e}  max |ref| {scale:.3e}  rel {err / scale:.3e}")
    assert err <= REL * scale
    # (3) the whole stack in fp64
    ol = [(f64(a), b.numpy().astype(np.float64), f64(c), d.numpy().astype(np.float64), ri)
          for (a, b, c, d), ri in zip(layers, tables)]
    exp = layer_stack_forward(f64(x), ol, pd, w.H, w.block)
    err, scale = np.abs(got - exp).max(), np.abs(exp).max()
    say(f"  whole stack: max err {err:.3e}  max |ref| {scale:.3e}  rel {err / scale:.3e}")
    assert err <= n_layers * REL * scale
