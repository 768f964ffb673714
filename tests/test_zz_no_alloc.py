"""The forward without allocation (bb_attn_forward_noalloc, through the C
ABI): the same bits as bb_attn_forward with a caller workspace, on two calls
in a row, the second with a smaller input (the library's scratch area keeps
the first call's partials, and nothing may depend on them); sizes beyond the
area are rejected before any launch."""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_bigbird_amd import binding as bb
from block_sparse_long_bigbird_amd.workloads import WORKLOADS, make_inputs, small

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    bb.lib()
    return torch.device("cuda:0")


def both_ways(w, dev):
    q, k, v, pad = make_inputs(w)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dpad = None if pad is None else pad.to(dev)
    dri = bb.upload_rand_idx(bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r), w.H, w.L,
                             w.block, w.r, dev)
    ref = torch.full_like(dq, float("nan"))
    ws = torch.full((bb.bb_attn_workspace_bytes(w.B, w.H, w.L, w.d, w.block),), 0xFF, dtype=torch.uint8,
                    device=dev)
    bb.bb_attn_forward(dq, dk, dv, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, ref, ws)
    got = torch.full_like(dq, float("nan"))
    say(f"  noalloc {w.name} B={w.B} H={w.H} L={w.L} block={w.block}")
    bb.bb_attn_forward_noalloc(dq, dk, dv, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_call_twice_second_smaller(dev):
    first = WORKLOADS["base_B4_H12_L4096_pad"]
    second = small("noalloc_small", B=1, H=2, L=9 * 64, block=64, r=2, pad="fixed", valid_len=9 * 64 - 40,
                   data_seed=41)
    for w in (first, second):
        ref, got = both_ways(w, dev)
        assert not torch.isnan(got).any().item()
        assert torch.equal(ref, got), f"{w.name}: max diff {(ref.float() - got.float()).abs().max().item()}"
    # and block 128 (the other kernel), smaller again
    third = small("noalloc_bs128", B=1, H=2, L=6 * 128, block=128, r=1, data_seed=42)
    ref, got = both_ways(third, dev)
    assert torch.equal(ref, got)


def test_noalloc_rejects_sizes_beyond_its_area(dev):
    B, H, L, block = 8, 16, 32768, 128            # partials of 277 MB > 64 MiB
    assert bb.bb_attn_workspace_bytes(B, H, L, 64, block) > bb.NOALLOC_SCRATCH_BYTES
    q = torch.empty((1, 1, 1, 64), dtype=torch.bfloat16, device=dev)   # never read: rejected first
    st = bb.lib().bb_attn_forward_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), None, None, B, H, L, 64,
                                          block, 0, q.data_ptr(), bb.BB_BF16, None)
    assert st == 5                                  # BB_ERR_WORKSPACE
    torch.cuda.synchronize()
