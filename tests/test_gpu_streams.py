"""The C ABI on streams other than the default one, and under HIP graph
capture: every entry point only enqueues kernels on the stream it is given
(no allocation, no memset, no synchronisation), so a call captured into a
graph must replay to the same bytes as the eager call.

Each graph is replayed several times with new inputs copied into its static
tensors between replays, eager work and synchronisations in between, and
every replay is compared bit for bit with an eager call on the same inputs.
Streams keep the default priority.
"""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import make_dout, make_inputs, make_layer_inputs, small

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()
    return torch.device("cuda:0")


W = small("streams_nb12_r3_pad", B=2, H=3, L=12 * 64, block=64, r=3, pad="per_seq_blocks",
          pad_lo_blocks=5, pad_hi_blocks=12, data_seed=81)


def inputs_on(dev, seed):
    w = small(W.name, B=W.B, H=W.H, L=W.L, block=W.block, r=W.r, pad=W.pad,
              pad_lo_blocks=W.pad_lo_blocks, pad_hi_blocks=W.pad_hi_blocks, data_seed=seed)
    q, k, v, pad = make_inputs(w)
    return [t.to(dev) for t in (q, k, v, pad, make_dout(w))]


def test_forward_on_side_stream_matches_default_stream(dev):
    q, k, v, pad, _ = inputs_on(dev, 81)
    ri = torch.from_numpy(bb.bb_rand_idx_build(W.rand_seed, W.H, W.L, W.block, W.r)).to(dev)
    ws = bb.alloc_workspace(W.B, W.H, W.L, W.d, W.block, dev)
    ref = torch.empty_like(q)
    bb.bb_attn_forward(q, k, v, pad, ri, W.B, W.H, W.L, W.d, W.block, W.r, ref, ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    out = torch.full_like(q, float("nan"))
    ws2 = bb.alloc_workspace(W.B, W.H, W.L, W.d, W.block, dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        bb.bb_attn_forward(q, k, v, pad, ri, W.B, W.H, W.L, W.d, W.block, W.r, out, ws2)
    s.synchronize()
    assert torch.equal(out, ref)


def test_forward_graph_replays_match_eager(dev):
    q, k, v, pad, _ = inputs_on(dev, 82)
    ri = torch.from_numpy(bb.bb_rand_idx_build(W.rand_seed, W.H, W.L, W.block, W.r)).to(dev)
    ws = bb.alloc_workspace(W.B, W.H, W.L, W.d, W.block, dev)
    out = torch.empty_like(q)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):        # warm-up on the capture stream
        bb.bb_attn_forward(q, k, v, pad, ri, W.B, W.H, W.L, W.d, W.block, W.r, out, ws)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bb.bb_attn_forward(q, k, v, pad, ri, W.B, W.H, W.L, W.d, W.block, W.r, out, ws)
    ws_e = bb.alloc_workspace(W.B, W.H, W.L, W.d, W.block, dev)
    for rep, seed in enumerate((83, 84, 85)):
        nq, nk, nv, npad, _ = inputs_on(dev, seed)
        q.copy_(nq), k.copy_(nk), v.copy_(nv), pad.copy_(npad)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(q)
        bb.bb_attn_forward(nq, nk, nv, npad, ri, W.B, W.H, W.L, W.d, W.block, W.r, ref, ws_e)
        torch.cuda.synchronize()
        say(f"  forward replay {rep}: equal={torch.equal(out, ref)}")
        assert torch.equal(out, ref), f"replay {rep}"


def test_backward_graph_replays_match_eager(dev):
    q, k, v, pad, dout = inputs_on(dev, 86)
    ri_h = bb.bb_rand_idx_build(W.rand_seed, W.H, W.L, W.block, W.r)
    ri = torch.from_numpy(ri_h).to(dev)
    off, rows = bb.bb_rand_idx_invert(ri_h, W.H, W.L, W.block, W.r)
    doff, drows = torch.from_numpy(off).to(dev), torch.from_numpy(rows).to(dev)
    ws = bb.alloc_workspace(W.B, W.H, W.L, W.d, W.block, dev)
    nbw = bb.bb_attn_backward_workspace_bytes(W.B, W.H, W.L, W.d, W.block)
    bws = torch.empty(nbw, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((W.B, W.H, W.L), dtype=torch.float32, device=dev)
    gq, gk, gv = (torch.empty_like(q) for _ in range(3))

    def call():
        bb.bb_attn_forward_lse(q, k, v, pad, ri, W.B, W.H, W.L, W.d, W.block, W.r, out, ws, lse)
        bb.bb_attn_backward(q, k, v, pad, ri, doff, drows, W.B, W.H, W.L, W.d, W.block, W.r, out, dout,
                            lse, gq, gk, gv, bws)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep, seed in enumerate((87, 88, 89)):
        nq, nk, nv, npad, ndo = inputs_on(dev, seed)
        q.copy_(nq), k.copy_(nk), v.copy_(nv), pad.copy_(npad), dout.copy_(ndo)
        for t in (gq, gk, gv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (gq, gk, gv)]
        call()                                   # eager, same static tensors
        torch.cuda.synchronize()
        eq = [torch.equal(a, b) for a, b in zip(got, (gq, gk, gv))]
        say(f"  backward replay {rep}: equal={eq}")
        assert all(eq), f"replay {rep}"


def test_layer_graph_replays_match_eager(dev):
    w = small("streams_layer_h256_nb8_r3_pad", B=2, H=4, L=8 * 64, block=64, r=3, pad="fixed",
              valid_len=8 * 64 - 50, data_seed=90)
    hid = w.H * w.d
    x, wq, bq, wo, bo, pad = (t.to(dev) for t in make_layer_inputs(w))
    ri = torch.from_numpy(bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)).to(dev)
    ws = torch.empty(bb.bb_layer_workspace_bytes(w.B, w.L, hid, w.H, w.block), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def call(xin, yout):
        bb.bb_layer_forward(xin, wq, bq, wo, bo, pad, ri, w.B, w.L, hid, w.H, w.block, w.r, yout, ws)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call(x, y)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(x, y)
    for rep in range(3):
        w2 = small(w.name, B=w.B, H=w.H, L=w.L, block=w.block, r=w.r, pad="fixed", valid_len=w.valid_len,
                   data_seed=92 + rep)
        nx = make_layer_inputs(w2)[0].to(dev)
        x.copy_(nx)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref = torch.empty_like(y)
        call(nx, ref)
        torch.cuda.synchronize()
        say(f"  layer replay {rep}: equal={torch.equal(got, ref)}")
        assert torch.equal(got, ref), f"replay {rep}"
