"""Pins for the oracle's attention layer (projections around the block-sparse
attention), CPU only:
  - identity projections with zero bias reduce the layer to the attention of
    the input split into heads (checked against the oracle's own, already
    pinned, attention, and per pair for one row);
  - the projections against torch.nn.functional.linear in float64 on the
    same weights (independent library code), with the attention between them;
  - linearity in the output projection: scaling W_o and b_o scales y;
  - layer_rows (selected output rows, used for the full-size GPU check) against
    the same torch.nn.functional.linear composition, row by row;
  - the layer stack: a layer whose q/k/v weights are zero attends with
    constant keys and values, so every row's output is the value bias, and
    the layer after it sees one constant row: closed forms for the whole
    stack, worked out with plain matrix-vector products; one layer is the
    layer itself; the order of the layers matters.
"""

import numpy as np
import torch

from oracle import attention_forward, layer_forward, layer_rows, layer_stack_forward


def sample_rand_idx(rng, H, nb, r):
    out = np.zeros((H, nb - 2, r), dtype=np.int32)
    for h in range(H):
        for i in range(1, nb - 1):
            cand = [j for j in range(1, nb - 1) if j not in (i - 1, i, i + 1)]
            out[h, i - 1] = rng.choice(cand, size=r, replace=False)
    return out


def case(seed, B=2, L=48, hid=12, H=3, block=4, r=2, padded=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, hid))
    w_qkv = rng.standard_normal((3 * hid, hid)) / np.sqrt(hid)
    b_qkv = rng.standard_normal(3 * hid) * 0.1
    w_o = rng.standard_normal((hid, hid)) / np.sqrt(hid)
    b_o = rng.standard_normal(hid) * 0.1
    ri = sample_rand_idx(rng, H, L // block, r)
    pad = None
    if padded:
        pad = np.ones((B, L), dtype=np.uint8)
        pad[:, L - 7:] = 0
    return x, w_qkv, b_qkv, w_o, b_o, pad, ri


def test_identity_projections_give_the_attention_of_the_heads():
    x, _, _, _, _, pad, ri = case(1)
    B, L, hid = x.shape
    H, d = 3, 4
    eye = np.eye(hid)
    y = layer_forward(x, np.concatenate([eye, eye, eye]), np.zeros(3 * hid), eye, np.zeros(hid),
                      pad, ri, H, 4)
    xh = x.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    att = attention_forward(xh, xh, xh, pad, ri, 4)
    assert np.abs(y - att.transpose(0, 2, 1, 3).reshape(B, L, hid)).max() <= 1e-12
    # one output row per pair: head 1 of row 0 (a global row: every key)
    b, t = 0, 0
    q = xh[b, 1, t]
    s = xh[b, 1] @ q / np.sqrt(d) - 10000.0 * (pad[b] == 0)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert np.abs(y[b, t, d:2 * d] - p @ xh[b, 1]).max() <= 1e-12


def test_projections_match_torch_linear():
    x, w_qkv, b_qkv, w_o, b_o, pad, ri = case(2)
    B, L, hid = x.shape
    H, d = 3, hid // 3
    t = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w_qkv), torch.tensor(b_qkv)).numpy()
    qkv = [t[..., i * hid:(i + 1) * hid].reshape(B, L, H, d).transpose(0, 2, 1, 3) for i in range(3)]
    att = attention_forward(*qkv, pad, ri, 4).transpose(0, 2, 1, 3).reshape(B, L, hid)
    exp = torch.nn.functional.linear(torch.tensor(att), torch.tensor(w_o), torch.tensor(b_o)).numpy()
    assert np.abs(layer_forward(x, w_qkv, b_qkv, w_o, b_o, pad, ri, H, 4) - exp).max() <= 1e-12


def test_output_projection_is_linear():
    x, w_qkv, b_qkv, w_o, b_o, pad, ri = case(3, padded=False)
    y1 = layer_forward(x, w_qkv, b_qkv, w_o, b_o, None, ri, 3, 4)
    y2 = layer_forward(x, w_qkv, b_qkv, 2.5 * w_o, 2.5 * b_o, None, ri, 3, 4)
    assert np.abs(y2 - 2.5 * y1).max() <= 1e-12


def test_layer_rows_match_torch_linear_composition():
    x, w_qkv, b_qkv, w_o, b_o, pad, ri = case(4)
    B, L, hid = x.shape
    H, d = 3, hid // 3
    t = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w_qkv), torch.tensor(b_qkv)).numpy()
    qkv = [t[..., i * hid:(i + 1) * hid].reshape(B, L, H, d).transpose(0, 2, 1, 3) for i in range(3)]
    att = attention_forward(*qkv, pad, ri, 4).transpose(0, 2, 1, 3).reshape(B, L, hid)
    exp = torch.nn.functional.linear(torch.tensor(att), torch.tensor(w_o), torch.tensor(b_o)).numpy()
    rows = np.array([0, 1, 3, 4, 17, 40, 44, 47])      # global blocks, band rows, padded rows
    got = layer_rows(x, w_qkv, b_qkv, w_o, b_o, pad, ri, H, 4, rows)
    assert got.shape == (B, len(rows), hid)
    assert np.abs(got - exp[:, rows]).max() <= 1e-12


def test_layer_stack_closed_form_after_a_constant_layer():
    """Layer 1 has zero q/k/v weights: its values are the bias b_v in every row,
    softmax weights sum to one, so its output row is c = b_v W_o1^T + b_o1 for
    every token.  Layer 2 then sees the constant row c: its values are
    c W_v2^T + b_v2 in every row, so y = (c W_v2^T + b_v2) W_o2^T + b_o2 for every
    token, whatever the masks and tables."""
    rng = np.random.default_rng(9)
    B, L, hid, H, block = 2, 48, 12, 3, 4
    x = rng.standard_normal((B, L, hid))
    pad = np.ones((B, L), dtype=np.uint8)
    pad[0, 30:] = 0
    layers = []
    for i in range(2):
        w_qkv = rng.standard_normal((3 * hid, hid)) / np.sqrt(hid)
        if i == 0:
            w_qkv[:] = 0.0
        layers.append((w_qkv, rng.standard_normal(3 * hid), rng.standard_normal((hid, hid)),
                       rng.standard_normal(hid), sample_rand_idx(rng, H, L // block, 2)))
    (_, b1, wo1, bo1, _), (w2, b2, wo2, bo2, _) = layers
    c = b1[2 * hid:] @ wo1.T + bo1
    v2 = c @ w2[2 * hid:].T + b2[2 * hid:]
    row = v2 @ wo2.T + bo2
    y = layer_stack_forward(x, layers, pad, H, block)
    assert np.abs(y - row[None, None, :]).max() <= 1e-10
    # one layer is the layer; the other order gives another result
    assert np.array_equal(layer_stack_forward(x, layers[:1], pad, H, block),
                          layer_forward(x, *layers[0][:4], pad, layers[0][4], H, block))
    assert np.abs(layer_stack_forward(x, layers[::-1], pad, H, block) - y).max() > 1e-3
