"""Pins for the fp64 oracle (CPU only).

The oracle is pinned to things other than itself: hand-derived golden
fixtures (tests/golden/), brute force on tiny inputs written as per-pair loops,
closed-form allowed-key counts, special cases that reduce to torch's
scaled_dot_product_attention, and invariants of softmax attention.
"""

import glob
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    attention_forward,
    attention_lse,
    attention_probs,
    block_adjacency,
    check_rand_idx,
    token_mask,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers ---

def sample_rand_idx(rng, H, nb, r):
    """A valid table drawn with numpy (independent of the library's builder)."""
    out = np.zeros((H, nb - 2, r), dtype=np.int32)
    for h in range(H):
        for i in range(1, nb - 1):
            cand = [j for j in range(1, nb - 1) if j not in (i - 1, i, i + 1)]
            out[h, i - 1] = rng.choice(cand, size=r, replace=False)
    return out


def allowed_pred(t, u, block, nb, rand_row_of):
    """Per-pair predicate, written from the prose of the pattern description."""
    bt, bu = t // block, u // block
    if bt == 0 or bt == nb - 1:          # global query blocks see everything
        return True
    if bu == 0 or bu == nb - 1:          # every query sees the global key blocks
        return True
    if abs(bt - bu) <= 1:                # 3-block band
        return True
    return bu in rand_row_of(bt)         # random blocks of this middle block


def brute_force(q, k, v, pad, rand_idx_h, block, query_mask=False):
    """Pure-Python loops with math.exp, one (batch, head).  query_mask: a pair
    gets the offset when its query or its key is padding."""
    L, d = len(q), len(q[0])
    nb = L // block
    rows = {i: set(int(x) for x in rand_idx_h[i - 1]) for i in range(1, nb - 1)}
    out = []
    for t in range(L):
        logits = []
        for u in range(L):
            if not allowed_pred(t, u, block, nb, lambda b: rows[b]):
                continue
            s = sum(q[t][c] * k[u][c] for c in range(d)) / math.sqrt(d)
            if pad is not None and (pad[u] == 0 or (query_mask and pad[t] == 0)):
                s += -10000.0
            logits.append((u, s))
        m = max(s for _, s in logits)
        w = [(u, math.exp(s - m)) for u, s in logits]
        z = sum(x for _, x in w)
        out.append([sum(x * v[u][c] for u, x in w) / z for c in range(d)])
    return np.array(out)


def rand_inputs(rng, B, H, L, d, scale=1.0):
    q = rng.standard_normal((B, H, L, d)) * scale
    k = rng.standard_normal((B, H, L, d)) * scale
    v = rng.standard_normal((B, H, L, d))
    return q, k, v


def sdpa(q, k, v, mask=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m).numpy()


def key_bias(pad, L):
    if pad is None:
        return np.zeros(L)
    return np.where(np.asarray(pad) == 0, -10000.0, 0.0)


# ------------------------------------------------------------ golden pins ---

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))))
def test_golden_fixture(path):
    with open(path) as f:
        g = json.load(f)
    L, block = g["L"], g["block"]
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    ri = np.array(g["rand_idx"], dtype=np.int64).reshape(1, L // block - 2, -1)
    for case in g["cases"]:
        pad = None if case["pad"] is None else np.array(case["pad"], dtype=np.uint8)[None]
        out = attention_forward(q, k, v, pad, ri, block)[0, 0]
        if "expected" in case:
            exp = np.array(case["expected"], dtype=np.float64)
        else:
            exp = np.tile(np.array(case["expected_row"]), (L, 1))
        np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)


# ------------------------------------------------------- brute-force pins ---

BRUTE_CASES = [
    # (block, nb, r, d, padded)
    (1, 3, 0, 1, False), (1, 5, 0, 2, True), (1, 6, 1, 3, False), (2, 6, 1, 2, True),
    (2, 7, 2, 3, False), (1, 8, 3, 2, True), (4, 5, 0, 3, True), (2, 9, 4, 1, False),
    (1, 10, 5, 2, True), (4, 4, 0, 2, False),
]


@pytest.mark.parametrize("block,nb,r,d,padded", BRUTE_CASES)
def test_brute_force_tiny(block, nb, r, d, padded):
    rng = np.random.default_rng(1000 + 7 * nb + block + 31 * r)
    B, H, L = 2, 2, nb * block
    q, k, v = rand_inputs(rng, B, H, L, d, scale=1.5)
    ri = sample_rand_idx(rng, H, nb, r)
    pad = None
    if padded:
        pad = np.ones((B, L), dtype=np.uint8)
        pad[0, L - max(1, L // 3):] = 0       # ragged, not block-aligned
        pad[1, rng.choice(L, size=max(1, L // 4), replace=False)] = 0
        pad[:, 0] = 1                          # keep a valid key in every row
    out = attention_forward(q, k, v, pad, ri, block)
    for b in range(B):
        for h in range(H):
            exp = brute_force(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(),
                              None if pad is None else pad[b].tolist(), ri[h], block)
            np.testing.assert_allclose(out[b, h], exp, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block,nb,r", [(1, 3, 0), (2, 4, 0), (1, 7, 2), (4, 6, 1), (2, 10, 5)])
def test_token_mask_matches_predicate(block, nb, r):
    rng = np.random.default_rng(nb * 13 + r)
    ri = sample_rand_idx(rng, 1, nb, r)[0]
    M = token_mask(block_adjacency(ri, nb), block)
    rows = {i: set(int(x) for x in ri[i - 1]) for i in range(1, nb - 1)}
    L = nb * block
    exp = np.array([[allowed_pred(t, u, block, nb, lambda b: rows[b]) for u in range(L)]
                    for t in range(L)])
    assert M.shape == (L, L)
    assert np.array_equal(M, exp)


# ------------------------------------------------------ closed-form pins ---

@pytest.mark.parametrize("block,nb,r", [(1, 3, 0), (3, 4, 0), (2, 5, 0), (2, 8, 3), (4, 12, 3),
                                        (1, 16, 11), (2, 64, 3)])
def test_allowed_counts_closed_form(block, nb, r):
    """Each middle row sees block*(band+globals deduped + r) keys; global rows see L."""
    rng = np.random.default_rng(nb + r)
    ri = sample_rand_idx(rng, 1, nb, r)[0]
    M = token_mask(block_adjacency(ri, nb), block)
    L = nb * block
    counts = M.sum(axis=1)
    for t in range(L):
        i = t // block
        if i in (0, nb - 1):
            assert counts[t] == L
        else:
            distinct = 5 - (i - 1 == 0) - (i + 1 == nb - 1)
            assert counts[t] == block * (distinct + r)
    # total attended pairs: 2*bs*L + bs^2 * [(nb-4)(5+r) + 2(4+r)]
    assert M.sum() == 2 * block * L + block * block * ((nb - 4) * (5 + r) + 2 * (4 + r))


def test_dense_when_every_block_is_covered():
    """nb in {3, 4} with r=0: every pair is allowed, so the result is dense attention."""
    rng = np.random.default_rng(5)
    for nb, block in [(3, 4), (4, 3), (3, 16)]:
        L, d = nb * block, 8
        q, k, v = rand_inputs(rng, 2, 3, L, d)
        ri = np.zeros((3, nb - 2, 0), dtype=np.int32)
        out = attention_forward(q, k, v, None, ri, block)
        np.testing.assert_allclose(out, sdpa(q, k, v), rtol=0, atol=1e-12)
        pad = np.ones((2, L), dtype=np.uint8)
        pad[0, -3:] = 0
        pad[1, 1] = 0
        out = attention_forward(q, k, v, pad, ri, block)
        bias = np.stack([key_bias(pad[b], L) for b in range(2)])[:, None, None, :]
        exp = sdpa(q, k, v, np.broadcast_to(bias, (2, 3, L, L)).copy())
        np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block,nb,r", [(4, 9, 2), (2, 16, 5), (8, 6, 1)])
def test_global_rows_are_dense_rows(block, nb, r):
    rng = np.random.default_rng(17 + nb)
    L, d, H = nb * block, 16, 2
    q, k, v = rand_inputs(rng, 1, H, L, d)
    ri = sample_rand_idx(rng, H, nb, r)
    out = attention_forward(q, k, v, None, ri, block)
    dense = sdpa(q, k, v)
    g = np.r_[0:block, L - block:L]
    np.testing.assert_allclose(out[:, :, g], dense[:, :, g], rtol=0, atol=1e-12)
    # and with padding: global rows equal dense attention with the -10000 key bias
    pad = np.ones((1, L), dtype=np.uint8)
    pad[0, L - block - 3:] = 0
    out = attention_forward(q, k, v, pad, ri, block)
    exp = sdpa(q, k, v, np.broadcast_to(key_bias(pad[0], L), (1, H, L, L)).copy())
    np.testing.assert_allclose(out[:, :, g], exp[:, :, g], rtol=0, atol=1e-12)


@pytest.mark.parametrize("block,nb", [(2, 6), (4, 8), (1, 11)])
def test_full_random_coverage(block, nb):
    """r = nb-5: interior rows see every block (dense rows); edge middle rows miss one block."""
    rng = np.random.default_rng(nb * 3)
    r = nb - 5
    L, d, H = nb * block, 8, 2
    q, k, v = rand_inputs(rng, 1, H, L, d)
    ri = sample_rand_idx(rng, H, nb, r)
    out = attention_forward(q, k, v, None, ri, block)
    dense = sdpa(q, k, v)
    inner = np.arange(2 * block, (nb - 2) * block)
    np.testing.assert_allclose(out[:, :, inner], dense[:, :, inner], rtol=0, atol=1e-12)
    for i in (1, nb - 2):      # negative control: these rows are not dense
        rows = np.arange(i * block, (i + 1) * block)
        assert np.abs(out[:, :, rows] - dense[:, :, rows]).max() > 1e-6


# ------------------------------------------------------------ invariants ---

def test_rows_sum_to_one():
    rng = np.random.default_rng(9)
    for block, nb, r in [(2, 7, 2), (4, 10, 3), (1, 12, 4)]:
        L = block * nb
        q, k, _ = rand_inputs(rng, 1, 1, L, 4, scale=3.0)
        ri = sample_rand_idx(rng, 1, nb, r)
        pad = (rng.random(L) > 0.3).astype(np.uint8)
        pad[0] = 1
        P = attention_probs(q[0, 0], k[0, 0], pad, block_adjacency(ri[0], nb), block)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (P[~token_mask(block_adjacency(ri[0], nb), block)] == 0).all()


def test_constant_v():
    rng = np.random.default_rng(10)
    block, nb, r = 4, 9, 3
    L = block * nb
    q, k, _ = rand_inputs(rng, 2, 2, L, 8, scale=2.0)
    v = np.full((2, 2, L, 8), 0.375)
    ri = sample_rand_idx(rng, 2, nb, r)
    pad = np.ones((2, L), dtype=np.uint8)
    pad[1, L // 2:] = 0
    out = attention_forward(q, k, v, pad, ri, block)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_over_allowed_valid_keys():
    rng = np.random.default_rng(11)
    block, nb, r = 3, 10, 2
    L = block * nb
    _, k, v = rand_inputs(rng, 1, 2, L, 5)
    q = np.zeros_like(k)
    ri = sample_rand_idx(rng, 2, nb, r)
    pad = np.ones((1, L), dtype=np.uint8)
    pad[0, 20:] = 0
    out = attention_forward(q, k, v, pad, ri, block)
    for h in range(2):
        rows = {i: set(int(x) for x in ri[h, i - 1]) for i in range(1, nb - 1)}
        for t in range(L):
            keys = [u for u in range(L)
                    if allowed_pred(t, u, block, nb, lambda b: rows[b]) and pad[0, u]]
            np.testing.assert_allclose(out[0, h, t], v[0, h, keys].mean(axis=0), rtol=0, atol=1e-12)


def test_padded_keys_do_not_matter():
    """Changing k/v at padded keys leaves every row unchanged (exp(-10000) == 0 in fp64)."""
    rng = np.random.default_rng(12)
    block, nb, r = 4, 12, 3
    L = block * nb
    q, k, v = rand_inputs(rng, 1, 2, L, 8)
    ri = sample_rand_idx(rng, 2, nb, r)
    pad = np.ones((1, L), dtype=np.uint8)
    pad[0, 30:] = 0
    pad[0, 7] = 0
    a = attention_forward(q, k, v, pad, ri, block)
    k2, v2 = k.copy(), v.copy()
    bad = pad[0] == 0
    k2[:, :, bad] = rng.standard_normal(k2[:, :, bad].shape) * 5
    v2[:, :, bad] = 1e6
    b = attention_forward(q, k2, v2, pad, ri, block)
    assert np.array_equal(a, b)


def test_all_padded_equals_unpadded():
    """pad == 0 everywhere shifts every logit by the same -10000: softmax is unchanged."""
    rng = np.random.default_rng(13)
    block, nb, r = 2, 8, 2
    L = block * nb
    q, k, v = rand_inputs(rng, 1, 2, L, 4)
    ri = sample_rand_idx(rng, 2, nb, r)
    a = attention_forward(q, k, v, None, ri, block)
    b = attention_forward(q, k, v, np.zeros((1, L), dtype=np.uint8), ri, block)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


def test_random_row_order_does_not_matter():
    rng = np.random.default_rng(14)
    block, nb, r = 2, 11, 4
    L = block * nb
    q, k, v = rand_inputs(rng, 1, 2, L, 4)
    ri = sample_rand_idx(rng, 2, nb, r)
    a = attention_forward(q, k, v, None, ri, block)
    ri2 = ri[:, :, ::-1].copy()
    b = attention_forward(q, k, v, None, ri2, block)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_rows_are_independent():
    """Evaluating rows in groups gives the same rows as all at once."""
    rng = np.random.default_rng(15)
    block, nb, r = 4, 9, 2
    L = block * nb
    q, k, v = rand_inputs(rng, 1, 1, L, 8)
    ri = sample_rand_idx(rng, 1, nb, r)
    a = attention_forward(q, k, v, None, ri, block, row_group=L)
    b = attention_forward(q, k, v, None, ri, block, row_group=5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)   # BLAS blocking may differ


# ------------------------------------------------- random-table checker ---

def test_check_rand_idx_accepts_valid_and_rejects_corrupt():
    rng = np.random.default_rng(16)
    H, nb, r, block = 3, 12, 3, 4
    L = nb * block
    ri = sample_rand_idx(rng, H, nb, r)
    check_rand_idx(ri, H, L, block, r)
    corrupt = []
    x = ri.copy(); x[1, 4, 1] = x[1, 4, 0]; corrupt.append(x)           # duplicate
    x = ri.copy(); x[0, 5, 2] = 6; corrupt.append(x)                    # own block (i=6)
    x = ri.copy(); x[0, 5, 2] = 5; corrupt.append(x)                    # band i-1
    x = ri.copy(); x[2, 0, 0] = 0; corrupt.append(x)                    # global block 0
    x = ri.copy(); x[2, 3, 1] = nb - 1; corrupt.append(x)               # global block nb-1
    x = ri.copy(); x[2, 3, 1] = nb + 3; corrupt.append(x)               # out of range
    x = ri.copy(); x[2, 3, 1] = -2; corrupt.append(x)                   # negative
    for x in corrupt:
        with pytest.raises(ValueError):
            check_rand_idx(x, H, L, block, r)
    with pytest.raises(ValueError):
        check_rand_idx(ri[:, :-1], H, L, block, r)                       # wrong shape
    with pytest.raises(ValueError):
        check_rand_idx(ri.astype(np.float64), H, L, block, r)            # not integer


def test_every_valid_table_enumerated_is_accepted():
    """Exhaustive: for nb=7, r=2 every combination per row is either valid or rejected correctly."""
    nb, r, block = 7, 2, 1
    for i in range(1, nb - 1):
        for combo in itertools.permutations(range(-1, nb + 1), r):
            ri = np.zeros((1, nb - 2, r), dtype=np.int64)
            for j in range(1, nb - 1):     # other rows: a fixed valid choice
                cand = [c for c in range(1, nb - 1) if c not in (j - 1, j, j + 1)]
                ri[0, j - 1] = cand[:r]
            ri[0, i - 1] = combo
            ok = all(1 <= c <= nb - 2 and c not in (i - 1, i, i + 1) for c in combo)
            if ok:
                check_rand_idx(ri, 1, nb * block, block, r)
            else:
                with pytest.raises(ValueError):
                    check_rand_idx(ri, 1, nb * block, block, r)


def test_check_rand_idx_cap_boundary():
    """The random-range cap (page "models 仓库中的 BigBird…", section "随机块掩码是如何生成的":
    random blocks are drawn only below token last_idx), pinned on both sides of its
    boundary with hand-picked values: with block 64, a block e lies inside the cap
    when its last token e*64 + 63 is below last_idx, i.e. e <= last_idx/64 - 1."""
    nb, block, r = 20, 64, 2
    L = nb * block

    def table(first_row_entries):
        ri = np.zeros((1, nb - 2, r), dtype=np.int64)
        for j in range(1, nb - 1):                 # every other row: blocks 1..5, off the window
            cand = [c for c in range(1, 6) if c not in (j - 1, j, j + 1)]
            ri[0, j - 1] = cand[:r]
        ri[0, 1] = first_row_entries               # row of middle block 2 (window 1, 2, 3)
        return ri

    for last_idx, inside, outside in [(640, 9, 10), (639, 8, 9), (650, 9, 10), (704, 10, 11),
                                      (384, 5, 6)]:
        check_rand_idx(table([inside, 4]), 1, L, block, r, last_idx=last_idx)
        with pytest.raises(ValueError, match="beyond token"):
            check_rand_idx(table([outside, 4]), 1, L, block, r, last_idx=last_idx)
        with pytest.raises(ValueError, match="beyond token"):
            check_rand_idx(table([4, outside]), 1, L, block, r, last_idx=last_idx)
    # no cap (last_idx = 0): the whole middle range, up to block nb - 2 = 18
    check_rand_idx(table([18, 4]), 1, L, block, r)


# --------------------------------------------- query-side (pair) masking ---
# Page "models 仓库中的 BigBird…", section on the random mask: the layer gets
# the blocked [B, L] mask and a band mask built from it by an einsum (query
# side x key side).  With query_mask the offset goes on every pair whose
# query or key is padding.

@pytest.mark.parametrize("block,nb,r,d", [(1, 5, 0, 2), (2, 6, 1, 2), (1, 8, 3, 2), (4, 5, 0, 3),
                                          (1, 10, 5, 2)])
def test_query_mask_brute_force_tiny(block, nb, r, d):
    rng = np.random.default_rng(5000 + 7 * nb + block + 31 * r)
    B, H, L = 2, 2, nb * block
    q, k, v = rand_inputs(rng, B, H, L, d, scale=1.5)
    ri = sample_rand_idx(rng, H, nb, r)
    pad = np.ones((B, L), dtype=np.uint8)
    pad[0, L - max(1, L // 3):] = 0
    pad[1, rng.choice(L, size=max(1, L // 4), replace=False)] = 0
    pad[:, 0] = 1
    out = attention_forward(q, k, v, pad, ri, block, query_mask=True)
    for b in range(B):
        for h in range(H):
            exp = brute_force(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), pad[b].tolist(), ri[h],
                              block, query_mask=True)
            np.testing.assert_allclose(out[b, h], exp, rtol=0, atol=1e-12)


def test_query_mask_valid_rows_unchanged_padded_rows_unmasked():
    """Closed forms of the pair rule: a valid query row is masked exactly as by
    the key-only rule (the same logits, bit for bit); on a padded query row
    every allowed logit gets the same offset, which cancels, so the row is
    the unmasked attention row; its log-sum-exp is the unmasked one - 10000."""
    rng = np.random.default_rng(77)
    B, H, nb, block, r, d = 2, 3, 9, 4, 3, 3
    L = nb * block
    q, k, v = rand_inputs(rng, B, H, L, d, scale=1.5)
    ri = sample_rand_idx(rng, H, nb, r)
    pad = np.ones((B, L), dtype=np.uint8)
    pad[0, 23:] = 0                                          # ragged suffix
    pad[1, rng.choice(L, size=12, replace=False)] = 0       # holes
    pad[:, 0] = 1
    pm = attention_forward(q, k, v, pad, ri, block, query_mask=True)
    km = attention_forward(q, k, v, pad, ri, block)
    um = attention_forward(q, k, v, None, ri, block)
    for b in range(B):
        valid = pad[b] != 0
        assert np.array_equal(pm[b][:, valid], km[b][:, valid])
        np.testing.assert_allclose(pm[b][:, ~valid], um[b][:, ~valid], rtol=0, atol=1e-9)
        assert np.abs(pm[b][:, ~valid] - km[b][:, ~valid]).max() > 1e-3   # the rule changes them
    lp = attention_lse(q, k, pad, ri, block, query_mask=True)
    lk = attention_lse(q, k, pad, ri, block)
    lu = attention_lse(q, k, None, ri, block)
    for b in range(B):
        valid = pad[b] != 0
        assert np.array_equal(lp[b][:, valid], lk[b][:, valid])
        np.testing.assert_allclose(lp[b][:, ~valid], lu[b][:, ~valid] - 10000.0, rtol=0, atol=1e-8)
