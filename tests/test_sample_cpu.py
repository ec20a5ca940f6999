"""Top-k sampling: pins of the oracle's Philox and uniform against numpy's own
Philox generator, of its float32 draw against the float64 definition of the
draw, and of its sampling by closed forms and statistics; host validation of
rtopk_sample_step (no launch)."""
import math

import numpy as np
import pytest

import oracle
from beam_search_top_amd import rtopk
from libutil import ensure_built


@pytest.mark.parametrize("key,ctr", [((0, 0), (1, 0, 0, 0)), ((123, 456), (1, 0, 0, 0)),
                                     ((2**64 - 1, 7), (5, 9, 0, 0)), ((42, 0), (2**64 - 1, 3, 1, 2))])
def test_philox_matches_numpy(key, ctr):
    # numpy's Philox bit generator is Philox4x64-10; it increments its counter
    # before each block, so the block of counter c comes from a state holding c - 1
    c = list(ctr)
    prev = [(c[0] - 1) % 2**64] + c[1:] if c[0] > 0 else [2**64 - 1, c[1] - 1] + c[2:]
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(prev, dtype=np.uint64))
    want = [int(v) for v in bg.random_raw(4)]
    assert list(oracle.philox4x64(ctr, key)) == want


def test_uniform_is_24_bit_in_unit_interval():
    us = [oracle.sample_uniform(7, r, 3) for r in range(2000)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(u) * 2**24 == int(float(u) * 2**24) for u in us)
    assert 0.45 < float(np.mean(us)) < 0.55


def _numpy_uniform(seed, row, step):
    """The sampling uniform from numpy's own Philox4x64-10 (not the oracle's):
    the 24 high bits of word 0 of the block with counter (row, step, 0, 0) and
    key (seed, 0), times 2^-24."""
    c = ((row + (step << 64)) - 1) % 2**256  # numpy increments the 256-bit counter before a block
    prev = [(c >> (64 * i)) & (2**64 - 1) for i in range(4)]
    bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64), counter=np.array(prev, dtype=np.uint64))
    return (int(bg.random_raw(1)[0]) >> 40) * 2.0**-24


@pytest.mark.parametrize("seed,step", [(0, 0), (11, 2), (2**63 + 5, 7), (123456789, 2**40)])
def test_uniform_is_the_high_bits_of_numpy_philox(seed, step):
    for row in (0, 1, 2, 17, 4095):
        assert float(oracle.sample_uniform(seed, row, step)) == _numpy_uniform(seed, row, step)


def _rows(R, V, seed, sigma=2.0):
    return np.random.default_rng(seed).normal(0, sigma, size=(R, V)).astype(np.float32)


def test_k1_and_cold_temperature_give_the_argmax():
    x = _rows(16, 300, 1)
    for s in (oracle.sample(x, oracle.F32, 1, 1.0, 5, 0), oracle.sample(x, oracle.F32, 8, 1e-6, 5, 0)):
        assert np.array_equal(s.tokens, np.argmax(x, axis=1))
    assert np.allclose(oracle.sample(x, oracle.F32, 1, 1.0, 5, 0).logprobs, 0.0)


def test_constant_rows_draw_uniformly_among_the_lowest_tokens():
    k = 10
    x = np.full((50, 64), 1.5, np.float32)
    s = oracle.sample(x, oracle.F32, k, 1.0, 11, 2)
    for r in range(50):
        u = _numpy_uniform(11, r, 2)  # equal weights: rank floor(u k) (u k is exact in float32 here)
        assert s.tokens[r] == min(int(math.floor(u * k)), k - 1)
    assert np.allclose(s.logprobs, -math.log(k))


def test_frequencies_follow_the_renormalised_top_k():
    V, k, tau = 40, 5, 0.7
    row = _rows(1, V, 3)[0]
    x = np.tile(row, (4000, 1))
    s = oracle.sample(x, oracle.F32, k, tau, 99, 0)
    top = np.argsort(-row, kind="stable")[:k]
    p = np.exp((row[top].astype(np.float64) - row[top[0]]) / tau)
    p /= p.sum()
    counts = np.array([(s.tokens == t).sum() for t in top])
    assert counts.sum() == 4000
    chi2 = float((((counts - 4000 * p) ** 2) / (4000 * p)).sum())
    assert chi2 < 20.5  # 4 degrees of freedom: p < 0.0005
    assert np.allclose(s.logprobs[:50], np.log(p[[list(top).index(t) for t in s.tokens[:50]]]), atol=1e-5)


@pytest.mark.parametrize("tau", [0.5, 1.0, 2.0])
def test_float32_draw_agrees_with_the_float64_definition(tau):
    # the definition in float64: exact top-k by (logit desc, index asc), scores
    # x - lse, weights exp((s_i - s_1) / tau), running sums in rank order, the
    # first rank whose sum exceeds u * S; the oracle's float32 decision may
    # differ only within float32 rounding of a boundary
    R, V, k, seed, draw = 3000, 60, 8, 5, 3
    x = _rows(R, V, 12, sigma=1.5)
    got = oracle.sample(x, oracle.F32, k, tau, seed, draw)
    near = 0
    for r in range(R):
        row = x[r].astype(np.float64)
        order = np.lexsort((np.arange(V), -row))[:k]
        m = row.max()
        lse = m + math.log(np.exp(row - m).sum())
        sc = row[order] - lse
        w = np.exp((sc - sc[0]) / tau)
        cs = np.cumsum(w)
        u = _numpy_uniform(seed, r, draw) * cs[-1]
        i = int(np.searchsorted(cs, u, side="right"))
        i = min(i, k - 1)
        margin = np.min(np.abs(cs - u)) / cs[-1]
        if margin < 1e-5:
            near += 1
            continue
        assert got.tokens[r] == order[i], (r, got.tokens[r], order[i])
        assert abs(got.logprobs[r] - math.log(w[i] / cs[-1])) < 1e-5
    assert near < R // 100


@pytest.fixture(scope="module")
def lib():
    ensure_built()
    return rtopk.load()


@pytest.mark.parametrize("args,msg", [
    ((0, 1, 4, 100, 4, 1.0, 0, 0, 0x1000, 0x2000), "NULL"),
    ((0x3000, 1, 4, 100, 4, 0.0, 0, 0, 0x1000, 0x2000), "temperature"),
    ((0x3000, 1, 4, 100, 4, float("nan"), 0, 0, 0x1000, 0x2000), "temperature"),
    ((0x3000, 1, 4, 100, 65, 1.0, 0, 0, 0x1000, 0x2000), "k=65"),
    ((0x3000, 1, 4, 100, 0, 1.0, 0, 0, 0x1000, 0x2000), "sizes"),
])
def test_sample_validation_rejects_before_launch(lib, args, msg):
    assert rtopk.rtopk_sample_step(*args, None) != 0
    assert msg in rtopk.rtopk_last_error()
