"""Cache refresh (beam reorder of a beam-major cache): pins of the oracle and
host-side validation of rtopk_beam_reorder (no launch)."""
import numpy as np
import pytest

import oracle
from beam_search_top_amd import rtopk
from libutil import ensure_built


def test_hand_worked_example():
    # 2 slabs, B=2, beam=3, 2-byte rows: row r of slab s holds bytes (10*s + r, 100 + 10*s + r).
    # Batch 0 keeps beams (2, 0, 2); batch 1 keeps (1, pad, 0): its padded row stays 0xEE.
    src = np.array([[[10 * s + r, 100 + 10 * s + r] for r in range(6)] for s in range(2)], dtype=np.uint8)
    before = np.full((2, 6, 2), 0xEE, dtype=np.uint8)
    ids = np.array([[2, 0, 2], [1, -1, 0]], dtype=np.int32)
    want = np.array([
        [[2, 102], [0, 100], [2, 102], [4, 104], [0xEE, 0xEE], [3, 103]],
        [[12, 112], [10, 110], [12, 112], [14, 114], [0xEE, 0xEE], [13, 113]],
    ], dtype=np.uint8)
    got = oracle.beam_reorder(src, before, ids, 2, 2, 3)
    assert np.array_equal(got, want)


def test_identity_and_inverse_permutation():
    rng = np.random.default_rng(3)
    nslabs, B, beam, R = 3, 4, 5, 7
    src = rng.integers(0, 256, size=(nslabs, B * beam, R), dtype=np.uint8)
    ident = np.tile(np.arange(beam, dtype=np.int32), (B, 1))
    assert np.array_equal(oracle.beam_reorder(src, np.zeros_like(src), ident, nslabs, B, beam), src)
    perm = np.stack([rng.permutation(beam) for _ in range(B)]).astype(np.int32)
    once = oracle.beam_reorder(src, np.zeros_like(src), perm, nslabs, B, beam)
    inv = np.argsort(perm, axis=1).astype(np.int32)
    assert np.array_equal(oracle.beam_reorder(once, np.zeros_like(src), inv, nslabs, B, beam), src)


def test_collapse_and_rows_stay_in_their_batch_element():
    rng = np.random.default_rng(4)
    nslabs, B, beam, R = 2, 3, 4, 5
    src = rng.integers(0, 256, size=(nslabs, B * beam, R), dtype=np.uint8)
    ids = rng.integers(-1, beam, size=(B, beam)).astype(np.int32)
    ids[0] = 2  # batch element 0: every beam continues old beam 2
    before = rng.integers(0, 256, size=src.shape, dtype=np.uint8)
    got = oracle.beam_reorder(src, before, ids, nslabs, B, beam)
    for s in range(nslabs):
        for j in range(beam):
            assert np.array_equal(got[s, j], src[s, 2])
        for b in range(B):
            for j in range(beam):
                i = ids[b, j]
                want = src[s, b * beam + i] if i >= 0 else before[s, b * beam + j]
                assert np.array_equal(got[s, b * beam + j], want)


@pytest.fixture(scope="module")
def lib():
    ensure_built()
    return rtopk.load()


@pytest.mark.parametrize("args,msg", [
    ((0, 0x10000, 1, 1, 1, 16, 0x2000, 1), "NULL"),
    ((0x1000, 0x900000, 0, 1, 1, 16, 0x2000, 1), "sizes"),
    ((0x1000, 0x900000, 1, 1, 0, 16, 0x2000, 1), "sizes"),
    ((0x1000, 0x900000, 1, 1, 4, 16, 0x2000, 3), "ld"),
    ((0x1000, 0x1010, 1, 1, 2, 16, 0x2000, 2), "overlap"),
    ((0x1000, 0x900000, 1, 1, 1, 0, 0x2000, 1), "sizes"),
    ((0x1000, 0x900000, 1 << 30, 1 << 20, 4, 1 << 20, 0x2000, 4), "overflows"),
])
def test_reorder_validation_rejects_before_launch(lib, args, msg):
    assert rtopk.rtopk_beam_reorder(*args, None) == rtopk.RTOPK_EINVAL
    assert msg in rtopk.rtopk_last_error()
