"""Pins for the oracle's backward pass and row log-sum-exp (CPU only).

Each pin comes from outside the oracle's backward formulas:
  - central finite differences of the oracle's forward (a different method:
    the derivative of the function the forward computes);
  - torch float64 autograd through a dense masked attention written here,
    per pair, from the pattern's prose (independent code and method);
  - exact invariants of softmax attention: every row of P sums to one, so the
    key-gradient sum vanishes and the value-gradient sum equals the
    output-gradient sum; a zero upstream gradient gives zero gradients;
  - the log-sum-exp against torch.logsumexp on the same independent logits,
    and the forward rebuilt from it;
  - pair masking (the offset when the query or the key is padding): autograd
    through the dense logits with the per-pair offset written here, and the
    closed forms that follow from the softmax -- a valid query row's dQ is the
    key-only masking's, a padded query row's dQ is the unmasked attention's.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward, attention_lse, check_rand_idx


def sample_rand_idx(rng, H, nb, r):
    """A valid table drawn with numpy (independent of the library's builder)."""
    out = np.zeros((H, nb - 2, r), dtype=np.int32)
    for h in range(H):
        for i in range(1, nb - 1):
            cand = [j for j in range(1, nb - 1) if j not in (i - 1, i, i + 1)]
            out[h, i - 1] = rng.choice(cand, size=r, replace=False)
    return out


def dense_mask_torch(L, block, rand_idx_h):
    """Allowed-pair mask [L, L] from the pattern's prose, per pair."""
    nb = L // block
    rows = {i: set(int(x) for x in rand_idx_h[i - 1]) for i in range(1, nb - 1)}
    m = torch.zeros(L, L, dtype=torch.bool)
    for t in range(L):
        bt = t // block
        for u in range(L):
            bu = u // block
            m[t, u] = (bt in (0, nb - 1) or bu in (0, nb - 1) or abs(bt - bu) <= 1
                       or (0 < bt < nb - 1 and bu in rows[bt]))
    return m


def torch_reference(q, k, v, pad, rand_idx, block, dout, query_mask=False):
    """float64 autograd through dense masked softmax attention (query_mask: the
    -10000 on a pair whose query or key is padding, else whose key is)."""
    B, H, L, d = q.shape
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    outs, lses = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(H):
            s = qt[b, h] @ kt[b, h].T / math.sqrt(d)
            if pad is not None:
                kp = pad[b] == 0
                off = (kp[None, :] | kp[:, None]) if query_mask else np.broadcast_to(kp[None, :], (L, L))
                s = s + torch.tensor(np.where(off, -10000.0, 0.0))
            s = s.masked_fill(~dense_mask_torch(L, block, rand_idx[h]), float("-inf"))
            ob.append(torch.softmax(s, dim=1) @ vt[b, h])
            lb.append(torch.logsumexp(s, dim=1))
        outs.append(torch.stack(ob))
        lses.append(torch.stack(lb))
    out = torch.stack(outs)
    (out * torch.tensor(dout)).sum().backward()
    return (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(),
            torch.stack(lses).detach().numpy(), out.detach().numpy())


def make_case(seed, B, H, nb, block, d, r, padded):
    rng = np.random.default_rng(seed)
    L = nb * block
    q, k, v, g = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    ri = sample_rand_idx(rng, H, nb, r)
    pad = None
    if padded:
        pad = np.ones((B, L), dtype=np.uint8)
        for b in range(B):
            pad[b, rng.integers(block, L):] = 0   # block 0 stays valid
    return q, k, v, g, ri, pad


@pytest.mark.parametrize("nb,block,r,padded", [(3, 2, 0, False), (6, 3, 1, False), (7, 2, 2, True)])
def test_backward_matches_central_differences(nb, block, r, padded):
    d = 3
    q, k, v, g, ri, pad = make_case(11 + nb, 1, 2, nb, block, d, r, padded)
    dq, dk, dv = attention_backward(q, k, v, pad, ri, block, g)

    def loss(**kw):
        args = dict(q=q, k=k, v=v)
        args.update(kw)
        return float((attention_forward(args["q"], args["k"], args["v"], pad, ri, block) * g).sum())

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(grad).max()), name


@pytest.mark.parametrize("nb,block,r,padded", [(8, 4, 3, True), (5, 8, 0, False), (10, 2, 5, True)])
def test_backward_and_lse_match_torch_autograd(nb, block, r, padded):
    q, k, v, g, ri, pad = make_case(100 + nb, 2, 2, nb, block, 4, r, padded)
    q = q * 2.0   # spread the logits
    tq, tk, tv, tlse, tout = torch_reference(q, k, v, pad, ri, block, g)
    dq, dk, dv = attention_backward(q, k, v, pad, ri, block, g)
    lse = attention_lse(q, k, pad, ri, block)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - b).max() <= 1e-10 * max(1.0, np.abs(b).max())
    assert np.abs(lse - tlse).max() <= 1e-9
    assert np.abs(attention_forward(q, k, v, pad, ri, block) - tout).max() <= 1e-12


def test_backward_invariants():
    q, k, v, g, ri, pad = make_case(7, 2, 3, 9, 4, 8, 2, True)
    dq, dk, dv = attention_backward(q, k, v, pad, ri, 4, g)
    # every row of P sums to one: sum_u dK_u = 0 and sum_u dV_u = sum_t dO_t
    assert np.abs(dk.sum(axis=2)).max() <= 1e-11
    assert np.abs(dv.sum(axis=2) - g.sum(axis=2)).max() <= 1e-11
    z = attention_backward(q, k, v, pad, ri, 4, np.zeros_like(g))
    assert all(np.abs(x).max() == 0.0 for x in z)


def test_backward_row_groups_do_not_change_the_result():
    q, k, v, g, ri, pad = make_case(3, 1, 2, 8, 4, 4, 2, True)
    a = attention_backward(q, k, v, pad, ri, 4, g)
    b = attention_backward(q, k, v, pad, ri, 4, g, row_group=5)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12


def test_lse_rebuilds_the_forward():
    """out_t = sum_u exp(s_tu - LSE_t) v_u over the allowed keys."""
    q, k, v, g, ri, pad = make_case(5, 1, 2, 6, 4, 4, 1, True)
    lse = attention_lse(q, k, pad, ri, 4)
    out = attention_forward(q, k, v, pad, ri, 4)
    L, d = q.shape[2], q.shape[3]
    for h in range(2):
        m = dense_mask_torch(L, 4, ri[h]).numpy()
        s = q[0, h] @ k[0, h].T / math.sqrt(d) + np.where(pad[0] == 0, -10000.0, 0.0)[None, :]
        p = np.where(m, np.exp(s - lse[0, h][:, None]), 0.0)
        assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-12
        assert np.abs(p @ v[0, h] - out[0, h]).max() <= 1e-12
    check_rand_idx(ri, 2, 24, 4, 1)


@pytest.mark.parametrize("nb,block,r", [(8, 4, 3), (10, 2, 5)])
def test_pair_masked_backward_matches_torch_autograd(nb, block, r):
    q, k, v, g, ri, pad = make_case(300 + nb, 2, 2, nb, block, 4, r, True)
    q = q * 2.0
    tq, tk, tv, tlse, tout = torch_reference(q, k, v, pad, ri, block, g, query_mask=True)
    dq, dk, dv = attention_backward(q, k, v, pad, ri, block, g, query_mask=True)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - b).max() <= 1e-10 * max(1.0, np.abs(b).max())
    assert np.abs(attention_lse(q, k, pad, ri, block, query_mask=True) - tlse).max() <= 1e-9


def test_pair_masked_backward_closed_forms():
    """dQ of a valid query row is the key-only masking's; dQ of a padded query
    row is the unmasked attention's (its offset is uniform and cancels); the
    softmax invariants still hold."""
    q, k, v, g, ri, pad = make_case(41, 2, 2, 9, 4, 4, 2, True)
    dq, dk, dv = attention_backward(q, k, v, pad, ri, 4, g, query_mask=True)
    dq_key, _, _ = attention_backward(q, k, v, pad, ri, 4, g)
    dq_none, _, _ = attention_backward(q, k, v, None, ri, 4, g)
    valid = (pad != 0)[:, None, :, None]
    assert np.abs(np.where(valid, dq - dq_key, 0.0)).max() <= 1e-12
    assert np.abs(np.where(valid, 0.0, dq - dq_none)).max() <= 1e-12
    assert (~valid).any() and np.abs(np.where(valid, 0.0, dq_key - dq_none)).max() > 1e-3
    assert np.abs(dk.sum(axis=2)).max() <= 1e-11
    assert np.abs(dv.sum(axis=2) - g.sum(axis=2)).max() <= 1e-11
