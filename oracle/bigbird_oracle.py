"""Plain fp64 CPU oracle for BigBird block-sparse self-attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, tables or helpers with the HIP
library; the two meet only through the seeded inputs handed to both.

Sources (the pages this follows; no code was available, only prose):
  [P2-pattern]  page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践"
                (TF Model Garden walkthrough), section
                "BigBird：从二次方注意力到线性稀疏注意力" -- the three-part pattern
                (3-block band, first/last block global, num_rand_blocks random
                blocks), the -10000 offset on masked logits and the softmax.
  [P2-randmask] same page, section "随机块掩码是如何生成的" -- random blocks are
                drawn from the block ids without the first and last block, the
                row's own window excluded; one table per head; the [B, L] input
                mask.
  [P4-method]   page "Big Bird: Transformers for Longer Sequences" (paper card),
                section "方法适配" -- global + window + random, block-level.

What it computes (the plainest reading of those passages; every reading the
pages leave open is listed in the design notes of the repository):
  nb = L / block, blk(t) = t // block, G = {0, nb-1},
  R_h(i) = set(rand_idx[h, i-1, :]) for middle block i in [1, nb-2].
  Allowed_h(t, u) <=> blk(t) in G  or  blk(u) in G  or  |blk(t)-blk(u)| <= 1
                      or  blk(u) in R_h(blk(t))
  s[b,h,t,u] = q.k / sqrt(d) - 10000 * [pad[b,u] == 0]      (allowed pairs)
  out[b,h,t] = sum_u softmax_u(s[b,h,t,:]) v[b,h,u]           (others: -inf)

Every step is a plain definition evaluated with numpy in float64: build the
block adjacency, expand it to the explicit token mask, dense masked softmax
attention.  Rows may be evaluated in groups (each row's softmax is
independent), which bounds host memory at long L; nothing else is blocked,
fused or reordered.

Backward (the gradient of the same function; the pages train this layer with
recomputation of the forward, [P2-pattern] page, section on the encoder's
recompute layer): with P the softmax above, O = P V, an upstream gradient dO
and s the scaled, biased logits,
  dV = P^T dO,  dP = dO V^T,  D_t = sum_d dO[t] O[t],
  dS = P * (dP - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d);
the pad offset is a constant and has no gradient.  The row log-sum-exp
LSE_t = log sum_u exp(s_tu) over the allowed keys is what a backward pass
needs from the forward to rebuild P.

Pins: see the test suite (brute force on tiny inputs, a hand-derived golden
fixture, closed-form allowed-key counts, dense/global special cases against
torch's scaled_dot_product_attention, invariants; for the backward, central
finite differences of the forward, float64 autograd of an independently
written dense masked attention, and exact invariants).
"""

from __future__ import annotations

import math

import numpy as np

MASK_OFFSET = -10000.0  # [P2-pattern]: masked logits get -10000 added


def num_blocks(L: int, block: int) -> int:
    if block <= 0 or L % block != 0:
        raise ValueError(f"L={L} is not a multiple of block={block}")
    nb = L // block
    if nb < 3:
        raise ValueError(f"need at least 3 blocks (two global + one middle), got {nb}")
    return nb


def check_rand_idx(rand_idx, H: int, L: int, block: int, r: int, last_idx: int = 0) -> None:
    """Raise ValueError unless rand_idx is a valid random-block table.

    [P2-randmask]: per head, one row per middle block (nb-2 rows), each row
    holding num_rand_blocks distinct block ids drawn from the middle blocks
    1..nb-2 with the row's own window {i-1, i, i+1} removed.  Row i-1 belongs
    to middle block i.  Order inside a row is not a constraint.
    last_idx > 0: the same page caps the random range at the first last_idx
    tokens; a block is inside the cap when it ends at or before that token.
    """
    nb = num_blocks(L, block)
    a = np.asarray(rand_idx)
    if a.shape != (H, nb - 2, r):
        raise ValueError(f"rand_idx shape {a.shape} != {(H, nb - 2, r)}")
    if r == 0:
        return
    if not np.issubdtype(a.dtype, np.integer):
        raise ValueError(f"rand_idx must be integer, got {a.dtype}")
    for h in range(H):
        for row in range(nb - 2):
            i = row + 1  # the middle block this row belongs to
            seen = set()
            for e in a[h, row].tolist():
                if not (1 <= e <= nb - 2):
                    raise ValueError(f"head {h} block {i}: random block {e} outside 1..{nb - 2}")
                if e in (i - 1, i, i + 1):
                    raise ValueError(f"head {h} block {i}: random block {e} inside the window")
                if e in seen:
                    raise ValueError(f"head {h} block {i}: random block {e} repeated")
                if last_idx > 0 and (e + 1) * block > last_idx:
                    raise ValueError(f"head {h} block {i}: random block {e} beyond token {last_idx}")
                seen.add(e)


def block_adjacency(rand_idx_h, nb: int) -> np.ndarray:
    """Block-level attention pattern of one head: bool [nb, nb], row = query block.

    [P2-pattern]: the first and last query blocks attend every key block; a
    middle block i attends its band {i-1, i, i+1}, the two global key blocks
    and its random blocks R_h(i).
    """
    A = np.zeros((nb, nb), dtype=bool)
    A[0, :] = True
    A[nb - 1, :] = True
    ri = np.asarray(rand_idx_h)
    for i in range(1, nb - 1):
        A[i, i - 1:i + 2] = True          # band
        A[i, 0] = True                    # global key blocks
        A[i, nb - 1] = True
        if ri.size:
            A[i, ri[i - 1]] = True        # random blocks of row i-1
    return A


def token_mask(adj: np.ndarray, block: int) -> np.ndarray:
    """Explicit L x L token mask: kron(adj, ones(block, block))."""
    return np.kron(adj, np.ones((block, block), dtype=bool)).astype(bool)


def _mask_rows(adj: np.ndarray, block: int, rows: np.ndarray) -> np.ndarray:
    """Rows `rows` of token_mask(adj, block), without building all L x L."""
    return np.repeat(adj[rows // block], block, axis=1)


def pair_masked(pad_b, rows, query_mask: bool) -> np.ndarray:
    """Which (query row, key) pairs get the offset: bool [len(rows), L].

    [P2-randmask]: the layer receives the blocked mask and a band mask made
    from it by an einsum, i.e. from the validity of the query side and of
    the key side.  Default (key side only): a pair is masked when its key
    is padding.  query_mask=True: when its query or its key is padding.
    """
    key_pad = np.asarray(pad_b) == 0
    m = np.broadcast_to(key_pad[None, :], (len(rows), key_pad.size))
    if query_mask:
        m = m | key_pad[np.asarray(rows)][:, None]
    return m


def attention_rows(q_bh, k_bh, v_bh, pad_b, adj, block: int, rows, query_mask: bool = False) -> np.ndarray:
    """Output rows `rows` of one (batch, head): fp64 [len(rows), d].

    q_bh/k_bh/v_bh: [L, d]; pad_b: [L] (nonzero = valid token) or None;
    adj: the head's block adjacency.  Dense masked softmax attention in fp64.
    query_mask: the offset on pairs whose query or key is padding (pair_masked).
    """
    q = np.asarray(q_bh, dtype=np.float64)
    k = np.asarray(k_bh, dtype=np.float64)
    v = np.asarray(v_bh, dtype=np.float64)
    L, d = k.shape
    rows = np.asarray(rows, dtype=np.int64)
    s = (q[rows] @ k.T) / math.sqrt(d)
    if pad_b is not None:
        s = s + MASK_OFFSET * pair_masked(pad_b, rows, query_mask).astype(np.float64)
    allowed = _mask_rows(adj, block, rows)
    s = np.where(allowed, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def attention_probs(q_bh, k_bh, pad_b, adj, block: int) -> np.ndarray:
    """Full probability matrix P [L, L] of one (batch, head); tiny inputs only."""
    q = np.asarray(q_bh, dtype=np.float64)
    k = np.asarray(k_bh, dtype=np.float64)
    L, d = k.shape
    s = (q @ k.T) / math.sqrt(d)
    if pad_b is not None:
        s = s + MASK_OFFSET * (np.asarray(pad_b) == 0).astype(np.float64)[None, :]
    s = np.where(token_mask(adj, block), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def attention_forward(q, k, v, pad_mask, rand_idx, block: int,
                      row_group: int = 4096, units=None, query_mask: bool = False) -> np.ndarray:
    """BigBird block-sparse attention forward in fp64.

    q, k, v: [B, H, L, d] (any real dtype; upcast to fp64 exactly as given);
    pad_mask: [B, L] (nonzero = valid) or None (no padding);
    rand_idx: [H, nb-2, r] integer table (validated first).
    units: optional iterable of (b, h) pairs to evaluate; other units are NaN.
    query_mask: pairs are masked when the query or the key is padding.
    Returns fp64 [B, H, L, d].
    """
    B, H, L, d = np.shape(q)
    nb = num_blocks(L, block)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    out = np.full((B, H, L, d), np.nan, dtype=np.float64)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    adjs = {}
    for b, h in units:
        if h not in adjs:
            adjs[h] = block_adjacency(rand_idx[h], nb)
        pad_b = None if pad_mask is None else np.asarray(pad_mask)[b]
        for r0 in range(0, L, row_group):
            rows = np.arange(r0, min(L, r0 + row_group))
            out[b, h, rows] = attention_rows(q[b, h], k[b, h], v[b, h], pad_b,
                                             adjs[h], block, rows, query_mask)
    return out


def _logits_rows(q, k, pad_b, adj, block: int, rows, query_mask: bool = False) -> np.ndarray:
    """Scaled, biased logits of rows `rows`, -inf off the pattern: fp64 [len(rows), L]."""
    L, d = k.shape
    s = (q[rows] @ k.T) / math.sqrt(d)
    if pad_b is not None:
        s = s + MASK_OFFSET * pair_masked(pad_b, rows, query_mask).astype(np.float64)
    return np.where(_mask_rows(adj, block, rows), s, -np.inf)


def attention_lse(q, k, pad_mask, rand_idx, block: int, units=None, query_mask: bool = False) -> np.ndarray:
    """Row log-sum-exp of the logits over the allowed keys: fp64 [B, H, L].

    LSE_t = log sum_u exp(s_tu), natural log, s as in the forward.
    units: optional (b, h) pairs to evaluate; other units are NaN.
    """
    B, H, L, d = np.shape(q)
    nb = num_blocks(L, block)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    out = np.full((B, H, L), np.nan, dtype=np.float64)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    for b, h in units:
        adj = block_adjacency(rand_idx[h], nb)
        pad_b = None if pad_mask is None else np.asarray(pad_mask)[b]
        s = _logits_rows(np.asarray(q[b, h], np.float64), np.asarray(k[b, h], np.float64),
                         pad_b, adj, block, np.arange(L), query_mask)
        m = s.max(axis=1, keepdims=True)
        out[b, h] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def attention_backward(q, k, v, pad_mask, rand_idx, block: int, dout, units=None,
                       row_group: int = 4096, query_mask: bool = False):
    """Gradients (dq, dk, dv) of sum(out * dout) for the forward above, fp64.

    q, k, v, dout: [B, H, L, d]; pad_mask [B, L] or None; rand_idx [H, nb-2, r].
    Follows the formulas in the module docstring, one (b, h) at a time; rows
    may be taken in groups (dK and dV are sums over rows, added group by group).
    units: optional (b, h) pairs to evaluate; other units are NaN.
    query_mask: the gradients of the pair-masked forward (pair_masked: the
    offset on pairs whose query or key is padding; page [P2], section
    "随机块掩码是如何生成的", the query-side and key-side masks).
    Returns three fp64 [B, H, L, d] arrays.
    """
    B, H, L, d = np.shape(q)
    nb = num_blocks(L, block)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    dq = np.full((B, H, L, d), np.nan, dtype=np.float64)
    dk = np.full((B, H, L, d), np.nan, dtype=np.float64)
    dv = np.full((B, H, L, d), np.nan, dtype=np.float64)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    for b, h in units:
        adj = block_adjacency(rand_idx[h], nb)
        pad_b = None if pad_mask is None else np.asarray(pad_mask)[b]
        dq[b, h], dk[b, h], dv[b, h] = attention_backward_unit(q[b, h], k[b, h], v[b, h], dout[b, h],
                                                               pad_b, adj, block, row_group, query_mask)
    return dq, dk, dv


def attention_backward_unit(q_bh, k_bh, v_bh, dout_bh, pad_b, adj, block: int, row_group: int = 4096,
                            query_mask: bool = False):
    """attention_backward for one (batch, head): q_bh, k_bh, v_bh, dout_bh [L, d];
    pad_b [L] or None; adj the head's block adjacency.  Returns (dq, dk, dv), fp64 [L, d]."""
    qb = np.asarray(q_bh, np.float64)
    kb = np.asarray(k_bh, np.float64)
    vb = np.asarray(v_bh, np.float64)
    gb = np.asarray(dout_bh, np.float64)
    L, d = kb.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.empty((L, d))
    dk = np.zeros((L, d))
    dv = np.zeros((L, d))
    for r0 in range(0, L, row_group):
        rows = np.arange(r0, min(L, r0 + row_group))
        s = _logits_rows(qb, kb, pad_b, adj, block, rows, query_mask)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)          # P, rows of the softmax
        o = p @ vb                                     # O
        g = gb[rows]                                   # dO
        dv += p.T @ g                                  # dV = P^T dO
        dp = g @ vb.T                                  # dP = dO V^T
        dsum = (g * o).sum(axis=1, keepdims=True)      # D = rowsum(dO * O)
        ds = p * (dp - dsum)                           # dS = P (dP - D)
        dq[rows] = (ds @ kb) * scale                   # dQ = dS K / sqrt(d)
        dk += (ds.T @ qb[rows]) * scale                # dK = dS^T Q / sqrt(d)
    return dq, dk, dv


def layer_forward(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, H: int, block: int) -> np.ndarray:
    """The attention layer around the block-sparse attention, fp64.

    [P2-pattern] page, the layer's construction: query, key and value come
    from input projections of the hidden states (key_dim = hidden / heads),
    and an output projection maps the concatenated heads back to hidden:
      [q | k | v] = x W_qkv^T + b_qkv      (W_qkv: [3*hidden, hidden], rows q, then k, then v)
      q, k, v split into H heads of d = hidden / H (head h = columns h*d .. h*d+d-1)
      o = attention(q, k, v) per head; concatenated back to [B, L, hidden]
      y = o W_o^T + b_o                     (W_o: [hidden, hidden])
    x: [B, L, hidden].  Returns fp64 [B, L, hidden].
    """
    x = np.asarray(x, dtype=np.float64)
    B, L, hid = x.shape
    d = hid // H
    proj = x @ np.asarray(w_qkv, np.float64).T + np.asarray(b_qkv, np.float64)
    def heads(t):                                        # [B, L, hid] -> [B, H, L, d]
        return t.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    q, k, v = (heads(proj[..., i * hid:(i + 1) * hid]) for i in range(3))
    o = attention_forward(q, k, v, pad_mask, rand_idx, block)
    o = o.transpose(0, 2, 1, 3).reshape(B, L, hid)
    return o @ np.asarray(w_o, np.float64).T + np.asarray(b_o, np.float64)


def layer_rows(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, H: int, block: int, rows) -> np.ndarray:
    """Rows `rows` (token indices, the same in every sequence) of layer_forward's
    output, fp64 [B, len(rows), hidden].

    The same steps as layer_forward: the projections of every token (keys and
    values need them all), attention_rows for the selected query rows of every
    head, and the output projection of those rows.
    """
    x = np.asarray(x, dtype=np.float64)
    B, L, hid = x.shape
    d = hid // H
    nb = num_blocks(L, block)
    rows = np.asarray(rows, dtype=np.int64)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    proj = x @ np.asarray(w_qkv, np.float64).T + np.asarray(b_qkv, np.float64)
    def heads(t):                                        # [B, L, hid] -> [B, H, L, d]
        return t.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    q, k, v = (heads(proj[..., i * hid:(i + 1) * hid]) for i in range(3))
    o = np.empty((B, len(rows), H, d))
    for h in range(H):
        adj = block_adjacency(rand_idx[h], nb)
        for b in range(B):
            pad_b = None if pad_mask is None else np.asarray(pad_mask)[b]
            o[b, :, h, :] = attention_rows(q[b, h], k[b, h], v[b, h], pad_b, adj, block, rows)
    return o.reshape(B, len(rows), hid) @ np.asarray(w_o, np.float64).T + np.asarray(b_o, np.float64)


def layer_stack_forward(x, layers, pad_mask, H: int, block: int) -> np.ndarray:
    """A stack of attention layers, fp64: h_0 = x, h_l = layer_forward(h_{l-1})
    with layer l's own weights and random-block table.

    [P2] page, the encoder's construction: the layers are stacked and each
    layer's random table is seeded with its index (the tables come in with
    the layers here).  layers: a sequence of (w_qkv, b_qkv, w_o, b_o,
    rand_idx), in order.  x: [B, L, hidden].  Returns fp64 [B, L, hidden].
    """
    h = np.asarray(x, dtype=np.float64)
    for w_qkv, b_qkv, w_o, b_o, rand_idx in layers:
        h = layer_forward(h, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, H, block)
    return h
