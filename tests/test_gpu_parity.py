"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max |gpu - oracle| over the compared outputs, padded query rows
included): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.
Small shapes and the full benchmark shapes are compared on every output (the
oracle runs unit by unit on a pool of host threads), with a NaN scan of the
whole output (the output buffer is NaN-poisoned first).  Only the tensors past
2^32 bytes are compared on sampled units and query blocks.
"""

import sys
import time

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import (STRESS_LONG, WORKLOADS, make_inputs,
                                                      make_inputs_device, small)
from oracle import attention_forward, attention_rows, block_adjacency
from oracle.parallel import forward_units, host_workers

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


def poisoned_workspace(w, dev):
    """Workspace filled with NaN bytes: any partial read before it is written shows up."""
    n = bb.bb_attn_workspace_bytes(w.B, w.H, w.L, w.d, w.block)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)


def run_gpu(w, dev, flags=bb.BB_LAUNCH_FUSED, inputs=None, ws=None):
    q, k, v, pad = inputs if inputs is not None else make_inputs(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
    out = torch.full_like(dq, float("nan"))
    if ws is None:
        ws = poisoned_workspace(w, dev)
    say(f"  launch {w.name} B={w.B} H={w.H} L={w.L} block={w.block} r={w.r} {w.dtype} flags={flags}")
    bb.bb_attn_forward(dq, dk, dv, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws, flags=flags)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (q, k, v, pad), ri


def f64(t):
    return t.to(torch.float64).numpy()


def compare_full(w, got, inputs, ri):
    q, k, v, pad = inputs
    exp = attention_forward(f64(q), f64(k), f64(v), None if pad is None else pad.numpy(), ri, w.block)
    assert not np.isnan(got).any(), "unwritten (NaN) outputs"
    err = np.abs(got - exp)
    nb = w.nb
    glob = np.zeros(w.L, dtype=bool)
    glob[: w.block] = True
    glob[(nb - 1) * w.block:] = True
    say(f"  max err global rows {err[:, :, glob].max():.3e}  middle rows "
        f"{err[:, :, ~glob].max() if (~glob).any() else 0:.3e}")
    assert err.max() <= TOL[w.dtype], err.max()


def sampled_rows(w, pad):
    nb = w.nb
    blocks = {0, 1, 2, nb // 2, nb - 3, nb - 2, nb - 1}
    if pad is not None:                      # a block in the padded region, and the boundary
        for b in range(w.B):
            valid = int(pad[b].sum())
            blocks.add(min(nb - 2, valid // w.block))
            blocks.add(max(1, min(nb - 2, valid // w.block + 3)))
    blocks = sorted(x for x in blocks if 0 <= x < nb)
    return np.concatenate([np.arange(x * w.block, (x + 1) * w.block) for x in blocks])


# ------------------------------------------------------------ small shapes ---

SMALL = [
    small("nb3_dense", B=2, H=3, L=3 * 64, block=64, r=0, data_seed=11),
    small("nb4_dense", B=1, H=2, L=4 * 64, block=64, r=0, data_seed=12),
    small("nb5", B=2, H=2, L=5 * 64, block=64, r=0, data_seed=13),
    small("nb6_r1", B=1, H=3, L=6 * 64, block=64, r=1, data_seed=14),
    small("nb9_r4_two_chunks", B=2, H=2, L=9 * 64, block=64, r=4, data_seed=15),
    small("nb17_r3_ragged_chunk", B=1, H=2, L=17 * 64, block=64, r=3, data_seed=16),
    small("nb12_r3_pad", B=3, H=2, L=12 * 64, block=64, r=3, pad="per_seq_blocks",
          pad_lo_blocks=4, pad_hi_blocks=12, data_seed=17),
    small("nb10_r2_pad_ragged", B=1, H=2, L=10 * 64, block=64, r=2, pad="fixed",
          valid_len=10 * 64 - 37, data_seed=18),
    small("nb20_r5_scale_small", B=1, H=2, L=20 * 64, block=64, r=5, value_scale=0.125, data_seed=19),
    small("bs128_nb3", B=1, H=2, L=3 * 128, block=128, r=0, data_seed=20),
    small("bs128_nb6_r1", B=2, H=1, L=6 * 128, block=128, r=1, data_seed=21),
    small("bs128_nb11_r4_pad", B=1, H=2, L=11 * 128, block=128, r=4, pad="fixed",
          valid_len=11 * 128 - 200, data_seed=22),
    small("fp32_nb3", B=1, H=2, L=3 * 64, block=64, r=0, dtype="fp32", data_seed=23),
    small("fp32_nb9_r3_pad", B=2, H=2, L=9 * 64, block=64, r=3, dtype="fp32", pad="fixed",
          valid_len=9 * 64 - 70, data_seed=24),
    small("fp32_bs128_nb7_r2", B=1, H=2, L=7 * 128, block=128, r=2, dtype="fp32", data_seed=25),
    small("outliers_unscaled", B=1, H=2, L=16 * 64, block=64, r=3, outlier_frac=0.02,
          outlier_mult=8.0, data_seed=26),
    # r = 16: middle units of 21 tiles run the tile loop in three trips
    # (8 + 8 + 5 steps), with padding; and the same in fp32 with block 128
    small("nb24_r16_pad_multi_trip", B=2, H=2, L=24 * 64, block=64, r=16, pad="per_seq_blocks",
          pad_lo_blocks=10, pad_hi_blocks=24, data_seed=27),
    small("fp32_bs128_nb22_r16", B=1, H=1, L=22 * 128, block=128, r=16, dtype="fp32", data_seed=28),
    # r = nb - 5, its largest value: every middle row attends every block
    # (lists of nb tiles), against the oracle's dense rows; bf16 with padding,
    # fp32, and bf16 at block 128
    small("nb30_r25_dense_rows_pad", B=1, H=2, L=30 * 64, block=64, r=25, pad="per_seq_blocks",
          pad_lo_blocks=12, pad_hi_blocks=30, data_seed=37),
    small("fp32_nb26_r21", B=1, H=2, L=26 * 64, block=64, r=21, dtype="fp32", data_seed=38),
    small("bs128_nb24_r19", B=1, H=2, L=24 * 128, block=128, r=19, data_seed=39),
    # pad masks with holes (mixed and fully padded subtiles between valid ones)
    small("nb10_r3_scattered_pad", B=2, H=2, L=10 * 64, block=64, r=3, pad="scattered", data_seed=29),
    small("bs128_nb7_r2_scattered_pad", B=1, H=2, L=7 * 128, block=128, r=2, pad="scattered",
          data_seed=30),
    small("fp32_nb8_r2_scattered_pad", B=1, H=2, L=8 * 64, block=64, r=2, dtype="fp32",
          pad="scattered", data_seed=32),
    # every key of every row padded: the offset is uniform per row and cancels
    small("nb8_r2_all_padded", B=2, H=2, L=8 * 64, block=64, r=2, pad="fixed", valid_len=0,
          data_seed=33),
    # logits tens of nats apart between tiles (5% of key rows x24, unscaled values):
    # rows whose later tiles exceed the first tile's max by far, recomputed exactly
    small("huge_logit_gaps", B=1, H=2, L=12 * 64, block=64, r=3, outlier_frac=0.05,
          outlier_mult=24.0, data_seed=35),
    small("huge_logit_gaps_bs128_pad", B=2, H=2, L=8 * 128, block=128, r=2, outlier_frac=0.05,
          outlier_mult=24.0, pad="fixed", valid_len=8 * 128 - 100, data_seed=36),
]
CASE = {w.name: w for w in SMALL}


@pytest.mark.parametrize("units", ["default", "ordinary"])
@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_full_parity(dev, w, units):
    """Every output against the oracle.  These shapes have too few ordinary
    work units to fill the device, so by default the key-group kernels split
    every query block over its key tiles (one to a few tiles per unit) and
    merge the chunks; BB_ORDINARY_UNITS runs the ordinary units instead."""
    say(f"case {w.name} units={units}")
    flags = bb.BB_ORDINARY_UNITS if units == "ordinary" else 0
    got, inputs, ri = run_gpu(w, dev, flags)
    compare_full(w, got, inputs, ri)


@pytest.mark.parametrize("w", [CASE["nb17_r3_ragged_chunk"], CASE["nb12_r3_pad"], CASE["bs128_nb11_r4_pad"],
                               CASE["fp32_bs128_nb7_r2"]],
                         ids=lambda w: w.name)
def test_split_launch_matches_fused_bitwise(dev, w):
    say(f"case split-vs-fused {w.name}")
    inputs = make_inputs(w)
    a, _, _ = run_gpu(w, dev, bb.BB_LAUNCH_FUSED | bb.BB_ORDINARY_UNITS, inputs=inputs)
    b, _, _ = run_gpu(w, dev, bb.BB_LAUNCH_SPLIT | bb.BB_ORDINARY_UNITS, inputs=inputs)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("w", [CASE["nb12_r3_pad"], CASE["bs128_nb11_r4_pad"]], ids=lambda w: w.name)
def test_two_phase_call_matches_single_call(dev, w):
    """BB_PHASE_UNITS then BB_PHASE_MERGE on the same stream == one full call, bit for bit."""
    say(f"case two-phase {w.name}")
    inputs = make_inputs(w)
    a, _, _ = run_gpu(w, dev, bb.BB_LAUNCH_FUSED, inputs=inputs)
    q, k, v, pad = inputs
    ri = torch.from_numpy(bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)).to(dev)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    for launch in (bb.BB_LAUNCH_FUSED, bb.BB_LAUNCH_SPLIT):
        out = torch.full_like(dq, float("nan"))
        ws = poisoned_workspace(w, dev)
        for phase in (bb.BB_PHASE_UNITS, bb.BB_PHASE_MERGE):
            bb.bb_attn_forward(dq, dk, dv, dpad, ri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws,
                               flags=launch | phase)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), a)


@pytest.mark.parametrize("w", [CASE["nb12_r3_pad"], CASE["bs128_nb11_r4_pad"]], ids=lambda w: w.name)
def test_timed_entry_matches_and_times(dev, w):
    """bb_attn_forward_timed: the same bits as the untimed call, for the whole call and
    for each phase, and its launch-recorded events bracket a positive duration."""
    say(f"case timed entry {w.name}")
    inputs = make_inputs(w)
    a, _, _ = run_gpu(w, dev, bb.BB_LAUNCH_FUSED, inputs=inputs)
    q, k, v, pad = inputs
    ri = torch.from_numpy(bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)).to(dev)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    stream = torch.cuda.current_stream(dev)
    for launch in (bb.BB_LAUNCH_FUSED, bb.BB_LAUNCH_SPLIT):
        for phases in ((0,), (bb.BB_PHASE_UNITS, bb.BB_PHASE_MERGE)):
            out = torch.full_like(dq, float("nan"))
            ws = poisoned_workspace(w, dev)
            evs = []
            for phase in phases:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for x in e:
                    x.record(stream)
                bb.bb_attn_forward(dq, dk, dv, dpad, ri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws,
                                   flags=launch | phase, events=e)
                evs.append(e)
            torch.cuda.synchronize()
            assert np.array_equal(out.float().cpu().numpy(), a)
            for e0, e1 in evs:
                assert e0.elapsed_time(e1) > 0.0


def test_bb_attn_forward_symbol_through_ctypes(dev):
    """bb_attn_forward itself, called through ctypes with raw device pointers
    (no binding wrapper), against the oracle on a padded multi-chunk case."""
    import ctypes
    w = CASE["nb12_r3_pad"]
    say(f"case ctypes bb_attn_forward {w.name}")
    q, k, v, pad = make_inputs(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    dq, dk, dv, dpad = q.to(dev), k.to(dev), v.to(dev), pad.to(dev)
    dri = torch.from_numpy(ri).to(dev)
    out = torch.full_like(dq, float("nan"))
    ws = poisoned_workspace(w, dev)
    P = ctypes.c_void_p
    st = bb.lib().bb_attn_forward(P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()),
                                  P(dpad.data_ptr()), P(dri.data_ptr()), w.B, w.H, w.L, w.d, w.block,
                                  w.r, P(out.data_ptr()), bb.BB_BF16, P(ws.data_ptr()), ws.numel(),
                                  P(torch.cuda.current_stream(dev).cuda_stream))
    assert st == bb.BB_OK, bb.bb_status_str(st)
    torch.cuda.synchronize()
    compare_full(w, out.float().cpu().numpy(), (q, k, v, pad), ri)


def test_deterministic_and_workspace_reuse(dev):
    """Same call twice gives identical bits; the workspace is ready for the next call,
    also for a different, smaller shape."""
    big = small("reuse_big", B=2, H=3, L=20 * 64, block=64, r=3, pad="fixed", valid_len=1200,
                data_seed=30)
    tiny = small("reuse_small", B=1, H=2, L=9 * 64, block=64, r=2, data_seed=31)
    say("case workspace reuse")
    ws = poisoned_workspace(big, dev)
    inputs = make_inputs(big)
    a, _, ri = run_gpu(big, dev, inputs=inputs, ws=ws)
    b, _, _ = run_gpu(big, dev, inputs=inputs, ws=ws)
    assert np.array_equal(a, b)
    compare_full(big, a, inputs, ri)
    c, inputs2, ri2 = run_gpu(tiny, dev, ws=ws)
    compare_full(tiny, c, inputs2, ri2)
    d, _, _ = run_gpu(big, dev, inputs=inputs, ws=ws)
    assert np.array_equal(a, d)


# ----------------------------------------------------- full benchmark shapes ---

def test_fp32_L1024_full(dev):
    w = WORKLOADS["fp32_B1_H2_L1024"]
    say(f"case {w.name}")
    got, inputs, ri = run_gpu(w, dev)
    compare_full(w, got, inputs, ri)


def compare_all_units(w, got, inputs, ri):
    """Every output of every (batch, head) unit against the oracle (evaluated
    unit by unit on a pool of host threads), plus the NaN scan."""
    q, k, v, pad = inputs
    assert not np.isnan(got).any(), "unwritten (NaN) outputs"
    t0 = time.perf_counter()
    exp = forward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                        None if pad is None else pad.numpy(), ri, w.block)
    err = np.abs(got - exp)
    glob = np.zeros(w.L, dtype=bool)
    glob[: w.block] = True
    glob[(w.nb - 1) * w.block:] = True
    say(f"  oracle on {w.B * w.H} units in {time.perf_counter() - t0:.1f} s ({host_workers()} threads); "
        f"max err global rows {err[:, :, glob].max():.3e}  middle rows {err[:, :, ~glob].max():.3e}")
    assert err.max() <= TOL[w.dtype], err.max()


@pytest.mark.parametrize("name", ["base_B4_H12_L4096_pad", "large_B8_H16_L4096",
                                  "pathx_B1_H8_L16384_pad", "long_B1_H12_L32768_bs128"])
def test_full_shape_parity_every_output(dev, name):
    """The benchmark shapes in the bench's launch configuration: every output of
    every (batch, head) against the oracle (persistent workgroups running long
    sequences of units across (batch, head), next-unit prefetch, per-XCD unit
    ranges -- paths that only shapes with more units than resident workgroups
    take)."""
    w = WORKLOADS[name]
    say(f"case {w.name}")
    got, inputs, ri = run_gpu(w, dev)
    compare_all_units(w, got, inputs, ri)


def test_stress_unscaled_outliers(dev):
    """32K tokens, block 128, unscaled values with x8 key outliers: the running max moves.
    Every output compared."""
    w = STRESS_LONG
    say(f"case {w.name}")
    got, inputs, ri = run_gpu(w, dev)
    compare_all_units(w, got, inputs, ri)


def test_tensors_over_4gib_sampled(dev):
    """64-bit addressing: q, k, v and out of 4.56 GB each, past 2^32 bytes (B 64,
    H 17, L 32768, block 128, r 4; global-row partials of 2.3 GB), drawn on the
    device.  The first, a middle and the last (batch, head) are compared on
    sampled query blocks."""
    w = small("big_B64_H17_L32768_bs128", B=64, H=17, L=32768, block=128, r=4,
              value_scale=0.125, data_seed=34)
    assert w.B * w.H * w.L * w.d * 2 > 2**32
    q, k, v = make_inputs_device(w, dev)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    out = torch.full_like(q, float("nan"))
    ws = poisoned_workspace(w, dev)
    say(f"  launch {w.name} ({q.numel() * 2 / 2**30:.2f} GiB per tensor)")
    bb.bb_attn_forward(q, k, v, None, torch.from_numpy(ri).to(dev), w.B, w.H, w.L, w.d, w.block,
                       w.r, out, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "unwritten (NaN) outputs"
    rows = sampled_rows(w, None)
    worst = 0.0
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, 7)]:
        adj = block_adjacency(ri[h], w.nb)
        exp = attention_rows(f64(q[b, h].cpu()), f64(k[b, h].cpu()), f64(v[b, h].cpu()), None, adj,
                             w.block, rows)
        got = out[b, h, rows].float().cpu().numpy()
        worst = max(worst, float(np.abs(got - exp).max()))
    say(f"  max err over 3 units x {len(rows)} rows: {worst:.3e}")
    assert worst <= TOL[w.dtype], worst


# --------------------------------------------------------------- error paths ---

def test_errors_raise_before_launch(dev):
    w = CASE["nb9_r4_two_chunks"]
    q, k, v, _ = make_inputs(w)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(dq)
    ri = torch.from_numpy(bb.bb_rand_idx_build(0, w.H, w.L, w.block, w.r)).to(dev)
    ws = bb.alloc_workspace(w.B, w.H, w.L, w.d, w.block, dev)
    with pytest.raises(bb.BBError, match="BB_ERR_WORKSPACE"):
        bb.bb_attn_forward(dq, dk, dv, None, ri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws[:64])
    with pytest.raises(ValueError, match="rand_idx has shape"):    # the binding's own check
        bb.bb_attn_forward(dq, dk, dv, None, ri, w.B, w.H, w.L, w.d, w.block, w.L // 64, out, ws)
    q32 = dq[..., :32].contiguous()                                # head dimension 32: the library's
    with pytest.raises(bb.BBError, match="BB_ERR_SHAPE"):
        bb.bb_attn_forward(q32, q32.clone(), q32.clone(), None, ri, w.B, w.H, w.L, 32, w.block, w.r,
                           torch.empty_like(q32), ws)
    bad = ri.clone()
    bad[0, 2, 0] = 3                                               # block 3 is in middle block 3's window
    with pytest.raises(bb.BBError, match="BB_ERR_RAND_IDX"):       # contents, checked once per table
        bb.bb_attn_forward(dq, dk, dv, None, bad, w.B, w.H, w.L, w.d, w.block, w.r, out, ws)
    with pytest.raises(bb.BBError, match="BB_ERR_ALIAS"):
        bb.bb_attn_forward(dq, dk, dv, None, ri, w.B, w.H, w.L, w.d, w.block, w.r, dq, ws)
    with pytest.raises(bb.BBError, match="BB_ERR_DTYPE"):
        bb.bb_attn_forward(dq.half(), dk.half(), dv.half(), None, ri, w.B, w.H, w.L, w.d, w.block,
                           w.r, out.half(), ws)
    torch.cuda.synchronize()


# ------------------------------------------- pad bytes other than 0 and 1 ---

def odd_pad_bytes(pad):
    """The same mask with every real token's byte replaced by 0x55 or 0xAA,
    alternating per 8-byte word: the AND of a 32-byte subtile's four words then
    has zero bytes even where no key is padding, so the kernels' all-valid
    pre-test (on that AND) falls through to their exact per-word test."""
    t = np.arange(pad.shape[1])
    vals = np.where((t // 8) % 2 == 0, 0x55, 0xAA).astype(np.uint8)
    return torch.from_numpy(np.where(pad.numpy() != 0, vals[None, :], 0).astype(np.uint8))


PADBYTE_CASES = [
    small("padbytes_nb8_r2_ragged", B=2, H=2, L=8 * 64, block=64, r=2, pad="fixed",
          valid_len=8 * 64 - 100, data_seed=71),
    small("padbytes_nb10_r3_seq", B=3, H=2, L=10 * 64, block=64, r=3, pad="per_seq_blocks",
          pad_lo_blocks=4, pad_hi_blocks=10, data_seed=72),
    small("padbytes_bs128_nb6_r1", B=2, H=2, L=6 * 128, block=128, r=1, pad="fixed",
          valid_len=6 * 128 - 200, data_seed=73),
    small("padbytes_fp32_nb8_r2", B=1, H=2, L=8 * 64, block=64, r=2, dtype="fp32", pad="fixed",
          valid_len=8 * 64 - 100, data_seed=74),
]


@pytest.mark.parametrize("flags", [bb.BB_LAUNCH_FUSED, bb.BB_ORDINARY_UNITS], ids=["default", "ordinary"])
@pytest.mark.parametrize("w", PADBYTE_CASES, ids=[w.name for w in PADBYTE_CASES])
def test_pad_bytes_other_than_one(dev, w, flags):
    """pad_mask is "nonzero = real token": valid bytes of 0x55 and 0xAA give
    the 0/1 mask's output bit for bit, and both match the oracle."""
    q, k, v, pad = make_inputs(w)
    ref, _, ri = run_gpu(w, dev, flags, inputs=(q, k, v, pad))
    got, _, _ = run_gpu(w, dev, flags, inputs=(q, k, v, odd_pad_bytes(pad)))
    assert not np.isnan(got).any()
    assert np.array_equal(got, ref)
    compare_full(w, got, (q, k, v, pad), ri)


# --------------------------------------------------- pair masking (flag) ---

QMASK_NAMES = ("nb12_r3_pad", "nb10_r2_pad_ragged", "bs128_nb11_r4_pad", "fp32_nb9_r3_pad",
               "nb24_r16_pad_multi_trip", "nb10_r3_scattered_pad", "bs128_nb7_r2_scattered_pad",
               "fp32_nb8_r2_scattered_pad", "nb8_r2_all_padded", "nb30_r25_dense_rows_pad")
QMASK_CASES = [w for w in SMALL if w.name in QMASK_NAMES]
assert len(QMASK_CASES) == len(QMASK_NAMES)


@pytest.mark.parametrize("w", QMASK_CASES, ids=[w.name for w in QMASK_CASES])
def test_query_mask_flag_matches_oracle(dev, w):
    """BB_QUERY_MASK: every output against the oracle's pair-masked attention;
    the rows of valid queries are bit-identical to the default (key-only) call."""
    say(f"case query mask {w.name}")
    inputs = make_inputs(w)
    plain, _, ri = run_gpu(w, dev, inputs=inputs)
    got, _, _ = run_gpu(w, dev, flags=bb.BB_QUERY_MASK, inputs=inputs)
    q, k, v, pad = inputs
    exp = attention_forward(f64(q), f64(k), f64(v), pad.numpy(), ri, w.block, query_mask=True)
    assert not np.isnan(got).any()
    err = np.abs(got - exp).max()
    valid = pad.numpy() != 0
    same = all(np.array_equal(got[b][:, valid[b]], plain[b][:, valid[b]]) for b in range(w.B))
    say(f"  max err {err:.3e}; valid query rows identical to the key-only call: {same}")
    assert err <= TOL[w.dtype]
    assert same


def test_query_mask_flag_full_shape(dev):
    """The padded 4 x 12 x 4096 shape with pair masking, every output."""
    w = WORKLOADS["base_B4_H12_L4096_pad"]
    say(f"case query mask {w.name}")
    inputs = make_inputs(w)
    got, _, ri = run_gpu(w, dev, flags=bb.BB_QUERY_MASK, inputs=inputs)
    q, k, v, pad = inputs
    exp = forward_units(q.float().numpy(), k.float().numpy(), v.float().numpy(), pad.numpy(), ri, w.block,
                        query_mask=True)
    assert not np.isnan(got).any()
    err = np.abs(got - exp).max()
    say(f"  max err {err:.3e}")
    assert err <= TOL[w.dtype]


def test_prepared_forward_matches_and_follows_its_inputs(dev):
    """PreparedForward (arguments checked once) gives bb_attn_forward's bits,
    and a second call after new values are written into q picks them up."""
    w = CASE["nb12_r3_pad"]
    say(f"case prepared forward {w.name}")
    inputs = make_inputs(w)
    a, _, _ = run_gpu(w, dev, inputs=inputs)
    q, k, v, pad = inputs
    ri = torch.from_numpy(bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)).to(dev)
    dq, dk, dv, dpad = q.to(dev), k.to(dev), v.to(dev), pad.to(dev)
    out = torch.full_like(dq, float("nan"))
    ws = poisoned_workspace(w, dev)
    call = bb.PreparedForward(dq, dk, dv, dpad, ri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws)
    call()
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), a)
    dq.copy_(dk)                                      # new query values, same storage
    call()
    b, _, _ = run_gpu(w, dev, inputs=(k, k, v, pad))
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), b)
