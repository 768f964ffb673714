"""GPU parity on seeded random small shapes: the forward with the row
log-sum-exp and the backward, through the C ABI, against the fp64 oracle,
each with the small-problem split (the default for most of these shapes)
and with the ordinary units (BB_ORDINARY_UNITS); the padded ones also with
pair masking (BB_QUERY_MASK).

The shapes are drawn once from a fixed seed (PCG64(2024)): block 64 or 128,
nb from 3 up, r from 0 to min(nb - 5, 16) (larger r: the explicit cases of
the parity and backward tests), B and H from
1 to 3, bf16 or fp32, and every padding mode (none, a fixed valid length
including zero, per-sequence block counts, scattered holes).  The case list
is printed by pytest's ids, so a failure names its shape.

Tolerances are those of the hand-picked cases: output 1e-5 (fp32) / 2e-2
(bf16) absolute on N(0,1) data; LSE 1e-5 / 5e-3; gradients 1e-4 / 2e-2 of
each tensor's largest oracle magnitude.
"""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import make_dout, make_inputs, small
from oracle import attention_backward, attention_forward, attention_lse

pytestmark = pytest.mark.gpu

OUT_TOL = {"fp32": 1e-5, "bf16": 2e-2}
LSE_TOL = {"fp32": 1e-5, "bf16": 5e-3}
GRAD_REL = {"fp32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw_cases(n: int = 24, seed: int = 2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        block = int(rng.choice([64, 128]))
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        nb = int(rng.integers(3, 26 if block == 64 else 14))
        r = int(rng.integers(0, min(max(nb - 5, 0), 16) + 1))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        L = nb * block
        pad = str(rng.choice(["none", "fixed", "per_seq_blocks", "scattered"]))
        kw = {}
        if pad == "fixed":
            kw["valid_len"] = int(rng.integers(0, L + 1))
        elif pad == "per_seq_blocks":
            lo = int(rng.integers(1, nb + 1))
            kw["pad_lo_blocks"], kw["pad_hi_blocks"] = lo, int(rng.integers(lo, nb + 1))
        name = f"rnd{i:02d}_{dtype}_bs{block}_nb{nb}_r{r}_B{B}H{H}_{pad}"
        cases.append(small(name, B=B, H=H, L=L, block=block, r=r, dtype=dtype, pad=pad,
                           data_seed=300 + i, rand_seed=i, **kw))
    return cases


CASES = draw_cases()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()
    return torch.device("cuda:0")


def f64(t):
    return t.to(torch.float64).numpy()


def run_case(dev, w, units, pair):
    """Forward with LSE and backward of case w through the C ABI against the
    oracle; pair: BB_QUERY_MASK (the oracle's pair-masked functions; the
    kernel's log-sum-exp of a padded query row leaves out the row's uniform
    -10000, so the oracle's gets +10000 on those rows)."""
    flags = (bb.BB_ORDINARY_UNITS if units == "ordinary" else 0) | (bb.BB_QUERY_MASK if pair else 0)
    q, k, v, pad = make_inputs(w)
    dout = make_dout(w)
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    off, rows = bb.bb_rand_idx_invert(ri, w.H, w.L, w.block, w.r)
    say(f"  {w.name} units={units} pair_masked={pair}")

    dq_, dk_, dv_ = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
    out = torch.full_like(dq_, float("nan"))
    lse = torch.full((w.B, w.H, w.L), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.full((bb.bb_attn_workspace_bytes(w.B, w.H, w.L, w.d, w.block),), 0xFF, dtype=torch.uint8,
                    device=dev)
    bb.bb_attn_forward_lse(dq_, dk_, dv_, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, out, ws, lse,
                           flags=flags)
    doff = torch.from_numpy(off).to(dev)
    drows = torch.from_numpy(rows).to(dev) if rows.size else None
    grads = [torch.full_like(dq_, float("nan")) for _ in range(3)]
    wsb = torch.full((bb.bb_attn_backward_workspace_bytes(w.B, w.H, w.L, w.d, w.block),), 0xFF,
                     dtype=torch.uint8, device=dev)
    bb.bb_attn_backward(dq_, dk_, dv_, dpad, dri, doff, drows, w.B, w.H, w.L, w.d, w.block, w.r, out,
                        dout.to(dev), lse, *grads, wsb, flags=flags)
    torch.cuda.synchronize()

    pn = None if pad is None else pad.numpy()
    got_out = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(got_out).any() and not np.isnan(got_lse).any(), "unwritten forward outputs"
    exp_out = attention_forward(f64(q), f64(k), f64(v), pn, ri, w.block, query_mask=pair)
    exp_lse = attention_lse(f64(q), f64(k), pn, ri, w.block, query_mask=pair)
    if pair:
        exp_lse = exp_lse + 10000.0 * (pn == 0)[:, None, :]
    e_out, e_lse = np.abs(got_out - exp_out).max(), np.abs(got_lse - exp_lse).max()
    say(f"    out err {e_out:.3e}  lse err {e_lse:.3e}")
    assert e_out <= OUT_TOL[w.dtype]
    assert e_lse <= LSE_TOL[w.dtype]

    exp = attention_backward(f64(q), f64(k), f64(v), pn, ri, w.block, f64(dout), query_mask=pair)
    for name, g, e in zip(("dq", "dk", "dv"), grads, exp):
        a = g.float().cpu().numpy()
        assert not np.isnan(a).any(), f"unwritten (NaN) {name}"
        err, scale = np.abs(a - e).max(), np.abs(e).max()
        say(f"    {name}: max err {err:.3e}  max |ref| {scale:.3e}")
        assert err <= GRAD_REL[w.dtype] * scale, name


@pytest.mark.parametrize("units", ["default", "ordinary"])
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_random_shape_forward_and_backward(dev, w, units):
    run_case(dev, w, units, pair=False)


PADDED = [w for w in CASES if w.pad != "none"]


@pytest.mark.parametrize("units", ["default", "ordinary"])
@pytest.mark.parametrize("w", PADDED, ids=[w.name for w in PADDED])
def test_random_shape_pair_masked(dev, w, units):
    """The padded cases again with BB_QUERY_MASK (a pair is masked when its
    query or its key is padding)."""
    run_case(dev, w, units, pair=True)
