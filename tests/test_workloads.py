"""The seeded input recipe (CPU only): what the workload generator promises
about its draws, so a change to it shows up here rather than as a shifted
benchmark or parity input."""

import numpy as np
import torch

from block_sparse_long_bigbird_amd.workloads import WORKLOADS, draw, make_inputs, small


def test_draws_are_reproducible_and_seed_dependent():
    w = small("w", B=2, H=2, L=8 * 64, block=64, r=2, pad="scattered", data_seed=5)
    a, b = draw(w), draw(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = draw(small("w", B=2, H=2, L=8 * 64, block=64, r=2, pad="scattered", data_seed=6))
    assert not np.array_equal(a[0], c[0]) and not np.array_equal(a[3], c[3])


def test_scattered_mask_has_its_own_stream():
    # q, k, v are the same draws whatever the pad mode
    kw = dict(B=2, H=2, L=8 * 64, block=64, r=2, data_seed=7)
    q0, k0, v0, _ = draw(small("a", pad="none", **kw))
    q1, k1, v1, pad = draw(small("b", pad="scattered", **kw))
    assert np.array_equal(q0, q1) and np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert pad.dtype == np.uint8 and set(np.unique(pad)) <= {0, 1}


def test_scattered_mask_shape():
    w = small("w", B=4, H=1, L=64 * 64, block=64, r=3, pad="scattered", data_seed=8)
    pad = draw(w)[3]
    span = 3 * w.block // 2
    for b in range(w.B):
        z = np.concatenate([[1], pad[b], [1]])
        edges = np.flatnonzero(np.diff(z))            # starts and ends of zero runs
        longest = (edges[1::2] - edges[0::2]).max()
        assert longest >= span                         # the padded span of 1.5 blocks
    assert abs(pad.mean() - 0.7 * (1 - span / w.L)) < 0.02


def test_per_sequence_block_padding():
    w = WORKLOADS["base_B4_H12_L4096_pad"]
    pad = draw(w)[3]
    valid = pad.sum(axis=1)
    assert np.all(valid % w.block == 0)
    assert np.all((valid >= w.pad_lo_blocks * w.block) & (valid <= w.pad_hi_blocks * w.block))
    for b in range(w.B):                              # a prefix of valid tokens
        assert np.all(pad[b, : valid[b]] == 1) and np.all(pad[b, valid[b]:] == 0)


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of finite float32 values, rounded to nearest, ties to even,
    written from the format's definition: keep the top 16 bits of the float32 word,
    adding half a unit of the kept last place minus one, plus that last bit (so an
    exact half rounds towards an even last bit)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    return ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_rne_reference_on_hand_picked_ties():
    # float32 words -> bfloat16 words, worked by hand: 1.0 is 0x3F80, the next
    # bfloat16 values up are 0x3F81 (1 + 2^-7) and 0x3F82 (1 + 2^-6)
    cases = {0x3F808000: 0x3F80,   # 1 + 2^-8: exact half, last bit 0 stays
             0x3F818000: 0x3F82,   # 1 + 3*2^-8: exact half, last bit 1 rounds up
             0x3F808001: 0x3F81,   # just above the half
             0x3F807FFF: 0x3F80,   # just below the half
             0xBF818000: 0xBF82,   # the same tie, negative
             0x3F80FFFF: 0x3F81}   # just below 0x3F81's upper half-way point
    words = np.array(list(cases), dtype=np.uint32)
    got = bf16_bits_rne(words.view(np.float32))
    assert got.tolist() == list(cases.values())


def test_inputs_rounded_once_to_nearest_even_bf16():
    w = small("w", B=1, H=2, L=4 * 64, block=64, r=0, value_scale=0.125, data_seed=9)
    q, k, v, _ = make_inputs(w)
    assert q.dtype == torch.bfloat16
    raw = draw(w)[:3]
    for got, x in zip((q, k, v), raw):
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), bf16_bits_rne(x))
    # ties occur among these draws only by chance: add explicit ties through the same path
    ties = np.array([0x3F808000, 0x3F818000, 0xBF818000, 0x3E018000], dtype=np.uint32).view(np.float32)
    conv = torch.from_numpy(ties.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(conv, bf16_bits_rne(ties))
