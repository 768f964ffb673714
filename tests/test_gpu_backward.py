"""GPU parity of the training entry points, through the C ABI, against the
fp64 oracle: the forward's row log-sum-exp (bb_attn_forward_lse) and the
backward pass (bb_attn_backward).

Tolerances:
  - LSE: 1e-5 (fp32 inputs); 5e-3 (bf16): the row sum is that of bf16-rounded
    probabilities (relative rounding <= 2^-9 each), so ln(l) moves by at most
    about 2^-9.
  - gradients: max |gpu - oracle| <= 2e-2 * max |oracle| per tensor for
    bf16 (1e-4 for fp32, where every operand and product is fp32).  Each product term carries bf16 operands (P, dS, dO, Q, K, V,
    relative rounding 2^-9 each, with fp32 accumulation) and the result is
    rounded to bf16 (2^-9); D is formed from the bf16 forward output.
Outputs and the workspace are poisoned (NaN / 0xFF) before every call, and
every output is scanned for NaN.
"""

import sys
import time

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import (WORKLOADS, make_dout, make_dout_device, make_inputs,
                                                      make_inputs_device, small)
from oracle import attention_backward, attention_forward, attention_lse
from oracle.parallel import backward_units

pytestmark = pytest.mark.gpu

LSE_TOL = {"fp32": 1e-5, "bf16": 5e-3}
GRAD_REL = {"bf16": 2e-2, "fp32": 1e-4}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()
    return torch.device("cuda:0")


def f64(t):
    return t.to(torch.float64).numpy()


def forward_lse(w, dev, inputs, ri, flags=0):
    q, k, v, pad = inputs
    dq_, dk_, dv_ = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
    out = torch.full_like(dq_, float("nan"))
    lse = torch.full((w.B, w.H, w.L), float("nan"), dtype=torch.float32, device=dev)
    n = bb.bb_attn_workspace_bytes(w.B, w.H, w.L, w.d, w.block)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    say(f"  forward_lse {w.name} B={w.B} H={w.H} L={w.L} block={w.block} r={w.r} {w.dtype} flags={flags}")
    bb.bb_attn_forward_lse(dq_, dk_, dv_, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws, lse,
                           flags=flags)
    torch.cuda.synchronize()
    return (dq_, dk_, dv_, dpad, dri), out, lse


LSE_CASES = [
    small("lse_nb5", B=2, H=2, L=5 * 64, block=64, r=0, data_seed=41),
    small("lse_nb12_r3_pad", B=3, H=2, L=12 * 64, block=64, r=3, pad="per_seq_blocks",
          pad_lo_blocks=4, pad_hi_blocks=12, data_seed=42),
    small("lse_nb17_r3", B=1, H=2, L=17 * 64, block=64, r=3, data_seed=43),
    small("lse_bs128_nb11_r4_pad", B=1, H=2, L=11 * 128, block=128, r=4, pad="fixed",
          valid_len=11 * 128 - 200, data_seed=44),
    small("lse_fp32_nb9_r3_pad", B=2, H=2, L=9 * 64, block=64, r=3, dtype="fp32", pad="fixed",
          valid_len=9 * 64 - 70, data_seed=45),
    small("lse_outliers_unscaled", B=1, H=2, L=16 * 64, block=64, r=3, outlier_frac=0.02,
          outlier_mult=8.0, data_seed=46),
]


@pytest.mark.parametrize("w", LSE_CASES, ids=[w.name for w in LSE_CASES])
def test_forward_lse_matches_oracle(dev, w):
    inputs = make_inputs(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    _, out, lse = forward_lse(w, dev, inputs, ri)
    q, k, v, pad = inputs
    pn = None if pad is None else pad.numpy()
    exp_out = attention_forward(f64(q), f64(k), f64(v), pn, ri, w.block)
    exp_lse = attention_lse(f64(q), f64(k), pn, ri, w.block)
    got_out = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(got_lse).any() and not np.isnan(got_out).any()
    e_out, e_lse = np.abs(got_out - exp_out).max(), np.abs(got_lse - exp_lse).max()
    say(f"  out err {e_out:.3e}  lse err {e_lse:.3e}")
    assert e_out <= {"fp32": 1e-5, "bf16": 2e-2}[w.dtype]
    assert e_lse <= LSE_TOL[w.dtype]


BWD_CASES = [
    small("bwd_nb3_dense", B=2, H=2, L=3 * 64, block=64, r=0, data_seed=51),
    small("bwd_nb5", B=1, H=2, L=5 * 64, block=64, r=0, data_seed=52),
    small("bwd_nb6_r1", B=1, H=3, L=6 * 64, block=64, r=1, data_seed=53),
    small("bwd_nb9_r4_two_chunks", B=2, H=2, L=9 * 64, block=64, r=4, data_seed=54),
    small("bwd_nb17_r3_ragged_chunk", B=1, H=2, L=17 * 64, block=64, r=3, data_seed=55),
    small("bwd_nb12_r3_pad", B=3, H=2, L=12 * 64, block=64, r=3, pad="per_seq_blocks",
          pad_lo_blocks=4, pad_hi_blocks=12, data_seed=56),
    small("bwd_nb10_r2_pad_ragged", B=1, H=2, L=10 * 64, block=64, r=2, pad="fixed",
          valid_len=10 * 64 - 37, data_seed=57),
    small("bwd_nb20_r5_scale_small", B=1, H=2, L=20 * 64, block=64, r=5, value_scale=0.125,
          data_seed=58),
    small("bwd_nb24_r16_pad_two_trips", B=2, H=2, L=24 * 64, block=64, r=16, pad="per_seq_blocks",
          pad_lo_blocks=10, pad_hi_blocks=24, data_seed=59),
    small("bwd_outliers_unscaled", B=1, H=2, L=16 * 64, block=64, r=3, outlier_frac=0.02,
          outlier_mult=8.0, data_seed=60),
    small("bwd_bs128_nb3", B=1, H=2, L=3 * 128, block=128, r=0, data_seed=61),
    small("bwd_bs128_nb6_r1", B=2, H=1, L=6 * 128, block=128, r=1, data_seed=62),
    small("bwd_bs128_nb11_r4_pad", B=1, H=2, L=11 * 128, block=128, r=4, pad="fixed",
          valid_len=11 * 128 - 200, data_seed=63),
    small("bwd_bs128_nb22_r16_two_trips", B=1, H=1, L=22 * 128, block=128, r=16, data_seed=64),
    # r = nb - 5: every middle row attends every block; the dK/dV lists of the
    # middle key blocks hold every query block
    small("bwd_nb30_r25_dense_rows_pad", B=1, H=2, L=30 * 64, block=64, r=25, pad="per_seq_blocks",
          pad_lo_blocks=12, pad_hi_blocks=30, data_seed=74),
    small("bwd_fp32_nb26_r21", B=1, H=2, L=26 * 64, block=64, r=21, dtype="fp32", data_seed=75),
    small("bwd_bs128_nb24_r19", B=1, H=2, L=24 * 128, block=128, r=19, data_seed=76),
    small("bwd_fp32_nb3", B=1, H=2, L=3 * 64, block=64, r=0, dtype="fp32", data_seed=66),
    small("bwd_fp32_nb9_r3_pad", B=2, H=2, L=9 * 64, block=64, r=3, dtype="fp32", pad="fixed",
          valid_len=9 * 64 - 70, data_seed=67),
    small("bwd_fp32_nb17_r3", B=1, H=2, L=17 * 64, block=64, r=3, dtype="fp32", data_seed=68),
    small("bwd_fp32_bs128_nb7_r2", B=1, H=2, L=7 * 128, block=128, r=2, dtype="fp32", data_seed=69),
    small("bwd_nb10_r3_scattered_pad", B=2, H=2, L=10 * 64, block=64, r=3, pad="scattered",
          data_seed=70),
    small("bwd_bs128_nb7_r2_scattered_pad", B=1, H=2, L=7 * 128, block=128, r=2, pad="scattered",
          data_seed=71),
    small("bwd_fp32_nb8_r2_scattered_pad", B=1, H=2, L=8 * 64, block=64, r=2, dtype="fp32",
          pad="scattered", data_seed=72),
    small("bwd_nb8_r2_all_padded", B=2, H=2, L=8 * 64, block=64, r=2, pad="fixed", valid_len=0,
          data_seed=73),
]


def run_backward(w, dev, inputs, ri, dout, flags=0):
    (dq_, dk_, dv_, dpad, dri), out, lse = forward_lse(w, dev, inputs, ri, flags)
    off, rows = bb.bb_rand_idx_invert(ri, w.H, w.L, w.block, w.r)
    doff = torch.from_numpy(off).to(dev)
    drows = torch.from_numpy(rows).to(dev) if rows.size else None
    g = dout.to(dev)
    gq, gk, gv = (torch.full_like(dq_, float("nan")) for _ in range(3))
    n = bb.bb_attn_backward_workspace_bytes(w.B, w.H, w.L, w.d, w.block)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    say(f"  backward {w.name}")
    bb.bb_attn_backward(dq_, dk_, dv_, dpad, dri, doff, drows, w.B, w.H, w.L, w.d, w.block, w.r,
                        out, g, lse, gq, gk, gv, ws, flags=flags)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (gq, gk, gv)]


def check_grads(got, exp, units=None, dtype="bf16"):
    worst = 0.0
    for name, a, b in zip(("dq", "dk", "dv"), got, exp):
        if units is not None:
            a = np.stack([a[bb_, h] for bb_, h in units])
            b = np.stack([b[bb_, h] for bb_, h in units])
        assert not np.isnan(a).any(), f"unwritten (NaN) {name}"
        scale = np.abs(b).max()
        err = np.abs(a - b).max()
        say(f"  {name}: max err {err:.3e}  max |ref| {scale:.3e}  rel {err / scale:.3e}")
        assert err <= GRAD_REL[dtype] * scale, name
        worst = max(worst, err / scale)
    return worst


def test_backward_pad_bytes_other_than_one(dev):
    """pad_mask is "nonzero = real token" in the backward too: valid bytes of
    0x55 and 0xAA (alternating per 8-byte word, so the AND of a subtile's pad
    words has zero bytes without any padded key) give the 0/1 mask's
    gradients bit for bit."""
    w = small("bwd_padbytes_nb8_r2", B=2, H=2, L=8 * 64, block=64, r=2, pad="fixed",
              valid_len=8 * 64 - 100, data_seed=75)
    q, k, v, pad = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    t = np.arange(w.L)
    vals = np.where((t // 8) % 2 == 0, 0x55, 0xAA).astype(np.uint8)
    odd = torch.from_numpy(np.where(pad.numpy() != 0, vals[None, :], 0).astype(np.uint8))
    ref = run_backward(w, dev, (q, k, v, pad), ri, dout)
    got = run_backward(w, dev, (q, k, v, odd), ri, dout)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(a).any(), name
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("units", ["default", "ordinary"])
@pytest.mark.parametrize("w", BWD_CASES, ids=[w.name for w in BWD_CASES])
def test_backward_matches_oracle(dev, w, units):
    """Every gradient of the small cases, with the small-problem split (every
    one of these shapes has fewer ordinary units than the split's threshold)
    and with the ordinary units (BB_ORDINARY_UNITS: the in-place middle blocks,
    the global blocks' split-K, tile lists longer than one trip)."""
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_backward(w, dev, inputs, ri, dout, flags=bb.BB_ORDINARY_UNITS if units == "ordinary" else 0)
    q, k, v, pad = inputs
    exp = attention_backward(f64(q), f64(k), f64(v), None if pad is None else pad.numpy(), ri,
                             w.block, f64(dout))
    check_grads(got, exp, dtype=w.dtype)


def test_backward_full_size_every_output(dev):
    """The benchmark shape (4 x 12 x 4096, padded): every gradient of every
    (batch, head) unit compared with the oracle (units spread over host threads)."""
    w = WORKLOADS["base_B4_H12_L4096_pad"]
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_backward(w, dev, inputs, ri, dout)
    q, k, v, pad = inputs
    t0 = time.perf_counter()
    exp = backward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(), pad.numpy(), ri, w.block,
                         dout.float().numpy())
    say(f"  oracle on {w.B * w.H} units in {time.perf_counter() - t0:.1f} s")
    check_grads(got, exp)


@pytest.mark.parametrize("name", ["fp32_B1_H2_L1024", "large_B8_H16_L4096", "long_B1_H12_L32768_bs128"])
def test_backward_other_benchmark_shapes_every_output(dev, name):
    """The other benchmark shapes (fp32 1 x 2 x 1024; 8 x 16 x 4096; 1 x 12 x
    32768 at block 128): every gradient of every (batch, head) unit against
    the oracle (units spread over host threads)."""
    w = WORKLOADS[name]
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_backward(w, dev, inputs, ri, dout)
    q, k, v, pad = inputs
    t0 = time.perf_counter()
    exp = backward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                         None if pad is None else pad.numpy(), ri, w.block, dout.float().numpy())
    say(f"  oracle on {w.B * w.H} units in {time.perf_counter() - t0:.1f} s")
    check_grads(got, exp, dtype=w.dtype)


def test_capped_random_range_forward_and_backward(dev):
    """A table whose random blocks all sit in the first 8 blocks (cap at token
    512): the inverted table then gives those key blocks long query lists
    (several trips of the dK/dV tile loop)."""
    w = small("capped_nb24_r3", B=1, H=2, L=24 * 64, block=64, r=3, pad="fixed",
              valid_len=24 * 64 - 90, data_seed=65)
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build_capped(3, w.H, w.L, w.block, w.r, 8 * 64)
    assert ri.max() <= 7
    off, _ = bb.bb_rand_idx_invert(ri, w.H, w.L, w.block, w.r)
    say(f"  longest inverted list: {int(np.diff(off, axis=1).max())} rows")
    got = run_backward(w, dev, inputs, ri, dout)
    q, k, v, pad = inputs
    exp = attention_backward(f64(q), f64(k), f64(v), pad.numpy(), ri, w.block, f64(dout))
    check_grads(got, exp)
    _, out, _ = forward_lse(w, dev, inputs, ri)
    e = np.abs(out.float().cpu().numpy() - attention_forward(f64(q), f64(k), f64(v), pad.numpy(), ri,
                                                              w.block)).max()
    say(f"  forward err {e:.3e}")
    assert e <= 2e-2


def test_backward_pathx_every_output(dev):
    """The Path-X shape (1 x 8 x 16384): blocks 240..255 are padding, the
    global key block 255 included (its dK and dV rows are zero; the padded
    query rows follow the same rule).  Every gradient of every (batch, head)
    unit compared with the oracle."""
    w = WORKLOADS["pathx_B1_H8_L16384_pad"]
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_backward(w, dev, inputs, ri, dout)
    q, k, v, pad = inputs
    t0 = time.perf_counter()
    exp = backward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(), pad.numpy(), ri, w.block,
                         dout.float().numpy())
    say(f"  oracle on {w.B * w.H} units in {time.perf_counter() - t0:.1f} s")
    check_grads(got, exp)
    # padded keys get no gradient
    valid = int(pad[0].sum())
    assert np.abs(got[1][0, :, valid:]).max() == 0.0 and np.abs(got[2][0, :, valid:]).max() == 0.0


def test_backward_tensors_over_4gib_sampled_units(dev):
    """64-bit addressing in both passes and the reduce: q, k, v, out, dout and
    the three gradients of 4.25 GiB each, past 2^32 bytes (B 64, H 17,
    L 32768, block 128, r 4), drawn on the device.  Gradients scanned for NaN
    on the device; the first and the last (batch, head) compared in full with
    the oracle."""
    w = small("big_bwd_B64_H17_L32768_bs128", B=64, H=17, L=32768, block=128, r=4,
              value_scale=0.125, data_seed=35)
    assert w.B * w.H * w.L * w.d * 2 > 2**32
    q, k, v = make_inputs_device(w, dev)
    g = make_dout_device(w, dev)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    dri = torch.from_numpy(ri).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    ws = bb.alloc_workspace(w.B, w.H, w.L, w.d, w.block, dev)
    say(f"  forward+lse {w.name} ({q.numel() * 2 / 2**30:.2f} GiB per tensor)")
    bb.bb_attn_forward_lse(q, k, v, None, dri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws, lse)
    off, rows = bb.bb_rand_idx_invert(ri, w.H, w.L, w.block, w.r)
    gq, gk, gv = (torch.full_like(q, float("nan")) for _ in range(3))
    n = bb.bb_attn_backward_workspace_bytes(w.B, w.H, w.L, w.d, w.block)
    bws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    say(f"  backward {w.name}")
    bb.bb_attn_backward(q, k, v, None, dri, torch.from_numpy(off).to(dev), torch.from_numpy(rows).to(dev),
                        w.B, w.H, w.L, w.d, w.block, w.r, out, g, lse, gq, gk, gv, bws)
    torch.cuda.synchronize()
    for name, t in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert not torch.isnan(t).any().item(), f"unwritten (NaN) {name}"
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        def sub(t):
            return f64(t[b:b + 1, h:h + 1].cpu())
        say(f"  oracle unit ({b}, {h})")
        exp = attention_backward(sub(q), sub(k), sub(v), None, ri[h:h + 1], w.block, sub(g))
        got = [t[b:b + 1, h:h + 1].float().cpu().numpy() for t in (gq, gk, gv)]
        check_grads(got, exp, dtype=w.dtype)


# ------------------------------------------------ pair masking (BB_QUERY_MASK) ---

QMASK_BWD_CASES = [c for c in BWD_CASES if c.pad != "none"]


@pytest.mark.parametrize("w", QMASK_BWD_CASES, ids=[w.name for w in QMASK_BWD_CASES])
def test_pair_masked_lse_and_backward_match_oracle(dev, w):
    """bb_attn_forward_lse_ex and bb_attn_backward_ex with BB_QUERY_MASK against
    the oracle's pair-masked forward, log-sum-exp and gradients.  The kernel's
    log-sum-exp of a padded query row leaves out the row's uniform -10000 (the
    header's reading), so the oracle's gets +10000 on those rows."""
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    q, k, v, pad = inputs
    pn = pad.numpy()
    _, out, lse = forward_lse(w, dev, inputs, ri, bb.BB_QUERY_MASK)
    exp_out = attention_forward(f64(q), f64(k), f64(v), pn, ri, w.block, query_mask=True)
    exp_lse = attention_lse(f64(q), f64(k), pn, ri, w.block, query_mask=True) + 10000.0 * (pn == 0)[:, None, :]
    got_out, got_lse = out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(got_lse).any() and not np.isnan(got_out).any()
    e_out, e_lse = np.abs(got_out - exp_out).max(), np.abs(got_lse - exp_lse).max()
    say(f"  out err {e_out:.3e}  lse err {e_lse:.3e}")
    assert e_out <= {"fp32": 1e-5, "bf16": 2e-2}[w.dtype]
    assert e_lse <= LSE_TOL[w.dtype]
    got = run_backward(w, dev, inputs, ri, dout, bb.BB_QUERY_MASK)
    exp = attention_backward(f64(q), f64(k), f64(v), pn, ri, w.block, f64(dout), query_mask=True)
    check_grads(got, exp, dtype=w.dtype)


def test_pair_masked_backward_full_size_every_output(dev):
    """The benchmark shape (4 x 12 x 4096, per-sequence padding) with pair
    masking: every gradient of every (batch, head) unit against the oracle."""
    w = WORKLOADS["base_B4_H12_L4096_pad"]
    inputs = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    got = run_backward(w, dev, inputs, ri, dout, bb.BB_QUERY_MASK)
    q, k, v, pad = inputs
    t0 = time.perf_counter()
    exp = backward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(), pad.numpy(), ri, w.block,
                         dout.float().numpy(), query_mask=True)
    say(f"  oracle on {w.B * w.H} units in {time.perf_counter() - t0:.1f} s")
    check_grads(got, exp)
