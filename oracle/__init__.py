"""CPU oracle for one beam-search decode step (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does. The arithmetic
lives in ``rtopk_oracle.c`` (plain C, float64): full log-softmax of every
alive beam, one full sort per batch element by (score desc, flat index asc),
as the LightSeq inference article's hierarchical-decoding passage states the
problem before its rewrite. This module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rtopk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, F16, BF16, F64 = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile liboracle.so with the host C compiler (gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", _SRC, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(L):
    """Declare the argument and result types of the oracle library's entry points."""
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    L.rtopk_oracle_step.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
    L.rtopk_oracle_step.restype = i32
    L.rtopk_oracle_lse.argtypes = [vp, i32, i64, i64, vp]
    L.rtopk_oracle_lse.restype = None
    L.rtopk_oracle_score_of.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32]
    L.rtopk_oracle_score_of.restype = f64
    L.rtopk_oracle_threshold.argtypes = [vp, i32, i64, i64, i32, i32, i64]
    L.rtopk_oracle_threshold.restype = f64
    L.rtopk_oracle_count_ge.argtypes = [vp, i32, i64, i64, f64]
    L.rtopk_oracle_count_ge.restype = i64
    L.rtopk_oracle_decode_f16.argtypes = [ctypes.c_uint16]
    L.rtopk_oracle_decode_f16.restype = f64
    L.rtopk_oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    L.rtopk_oracle_decode_bf16.restype = f64
    L.rtopk_oracle_lmhead_logits.argtypes = [vp, vp, i64, i64, i64, vp]
    L.rtopk_oracle_lmhead_logits.restype = None
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def _logits(x, dtype):
    want = {F32: np.float32, F16: np.float16, BF16: np.uint16, F64: np.float64}[dtype]
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"logits dtype {x.dtype} does not match code {dtype}")
    return x


class Result:
    """Oracle output for one step: [B, k] beam/token/score, fp64 scores, [B, beam] lse."""

    def __init__(self, beam_ids, token_ids, scores, scores64, lse):
        self.beam_ids, self.token_ids, self.scores = beam_ids, token_ids, scores
        self.scores64, self.lse = scores64, lse


def step(logits, dtype, alive, finished, k, eos_id=2, nthreads=1) -> Result:
    """Run the oracle on host arrays logits [B, beam, V], alive [B, beam], finished [B, beam] or None."""
    L = _load()
    x = _logits(logits, dtype)
    B, beam, V = x.shape
    alive = np.ascontiguousarray(alive, dtype=np.float32).reshape(B, beam)
    fin = None if finished is None else np.ascontiguousarray(finished, dtype=np.uint8).reshape(B, beam)
    ob = np.empty((B, k), np.int32)
    ot = np.empty((B, k), np.int32)
    os_ = np.empty((B, k), np.float32)
    o64 = np.empty((B, k), np.float64)
    lse = np.empty((B, beam), np.float64)
    rc = L.rtopk_oracle_step(_ptr(x), dtype, _ptr(alive), _ptr(fin), B, beam, V, k, eos_id,
                             _ptr(ob), _ptr(ot), _ptr(os_), _ptr(o64), _ptr(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"rtopk_oracle_step failed with status {rc}")
    return Result(ob, ot, os_, o64, lse)


def step_of(s, nthreads=1) -> Result:
    """Oracle on a ``synth.Step``."""
    return step(s.logits, s.dtype, s.alive, s.finished, s.k, s.eos_id, nthreads)


def lse(logits, dtype) -> np.ndarray:
    """float64 log-sum-exp of every row of logits [..., V]."""
    x = _logits(logits, dtype)
    V = x.shape[-1]
    nrows = x.size // V
    out = np.empty(nrows, np.float64)
    _load().rtopk_oracle_lse(_ptr(x), dtype, nrows, V, _ptr(out))
    return out.reshape(x.shape[:-1])


def score_of(logits, dtype, alive, finished, lse_, eos_id, b, j, t) -> float:
    """The oracle's float64 score of pair (b, j, t); -inf for non-candidates and padding."""
    x = _logits(logits, dtype)
    B, beam, V = x.shape
    alive = np.ascontiguousarray(alive, dtype=np.float32)
    fin = None if finished is None else np.ascontiguousarray(finished, dtype=np.uint8)
    lse_ = np.ascontiguousarray(lse_, dtype=np.float64)
    return _load().rtopk_oracle_score_of(_ptr(x), dtype, _ptr(alive), _ptr(fin), _ptr(lse_),
                                         B, beam, V, eos_id, int(b), int(j), int(t))


def threshold(x, dtype, ngroups, k, offset=0, base=0, n=None) -> float:
    """R-top-k of x[base:base+n] with element i in group (i + offset) mod ngroups."""
    x = _logits(x, dtype)
    n = x.size - base if n is None else n
    return _load().rtopk_oracle_threshold(_ptr(x), dtype, base, n, ngroups, k, offset)


def count_ge(x, dtype, T, base=0, n=None) -> int:
    x = _logits(x, dtype)
    n = x.size - base if n is None else n
    return int(_load().rtopk_oracle_count_ge(_ptr(x), dtype, base, n, float(T)))


def decode_f16(code: int) -> float:
    return _load().rtopk_oracle_decode_f16(int(code))


def decode_bf16(code: int) -> float:
    return _load().rtopk_oracle_decode_bf16(int(code))


def lmhead_logits(x_bits, w_bits):
    """float64 logits [M, V] of the LM head: x [M, H] hidden states and w
    [V, H] output projection as bfloat16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, H = x.shape
    V, H2 = w.shape
    if H != H2:
        raise ValueError("x and w disagree on H")
    out = np.empty((M, V), np.float64)
    _load().rtopk_oracle_lmhead_logits(_ptr(x), _ptr(w), M, V, H, _ptr(out))
    return out


def lmhead_step(x_bits, w_bits, alive, finished, beam, k, eos_id=2, nthreads=1) -> Result:
    """The fused LM-head step by its definition: the float64 logits of
    lmhead_logits, then the step oracle on them (rows m = b * beam + j)."""
    logits = lmhead_logits(x_bits, w_bits)
    M, V = logits.shape
    return step(logits.reshape(M // beam, beam, V), F64, alive, finished, k, eos_id, nthreads)


def beam_reorder(src, dst_before, beam_ids, nslabs, B, beam):
    """Cache refresh by its definition: once the selection has chosen, for
    batch element b, new beam j as a continuation of old beam beam_ids[b][j],
    the decoder's cache rows follow their beams (the LightSeq inference
    article ends the decode step with this cache update, after the
    hierarchical selection). In every slab s (a layer's keys or values), row
    b*beam + j of the result is row b*beam + beam_ids[b][j] of src; an id
    outside [0, beam) (padding) leaves the row of dst_before. Arrays are raw
    bytes, [nslabs][B*beam][row_bytes]; returns a new array."""
    src = np.asarray(src, dtype=np.uint8).reshape(nslabs, B, beam, -1)
    out = np.array(dst_before, dtype=np.uint8, copy=True).reshape(nslabs, B, beam, -1)
    ids = np.asarray(beam_ids)
    for b in range(B):
        for j in range(beam):
            i = int(ids[b, j])
            if 0 <= i < beam:
                out[:, b, j, :] = src[:, b, i, :]
    return out.reshape(nslabs, B * beam, -1)


# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011), from its definition:
# round constants, Weyl key increments, ten rounds.
_PH_M0, _PH_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_PH_W0, _PH_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
_M64 = (1 << 64) - 1


def philox4x64(counter, key, rounds=10):
    """The four 64-bit words of Philox4x64 for a 4-word counter and 2-word key."""
    c0, c1, c2, c3 = (int(v) & _M64 for v in counter)
    k0, k1 = (int(v) & _M64 for v in key)
    for _ in range(rounds):
        p0, p1 = _PH_M0 * c0, _PH_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0), p1 & _M64, ((p0 >> 64) ^ c3 ^ k1), p0 & _M64
        k0, k1 = (k0 + _PH_W0) & _M64, (k1 + _PH_W1) & _M64
    return c0, c1, c2, c3


def sample_uniform(seed, row, step):
    """u in [0, 1): the 24 high bits of word 0 of Philox4x64-10 with counter
    (row, step, 0, 0) and key (seed, 0), times 2^-24 (exact in float32)."""
    return np.float32((philox4x64((row, step, 0, 0), (seed, 0))[0] >> 40) * 2.0 ** -24)


class Sample:
    """Oracle output of top-k sampling: tokens [R], log-probabilities [R]
    (float64), and each row's decision margin |u*S - C_j| / S at the nearest
    cumulative sum boundary (float32 decisions within a few ulps of a boundary
    may go either way in another implementation)."""

    def __init__(self, tokens, logprobs, margins, topk_tokens):
        self.tokens, self.logprobs, self.margins, self.topk_tokens = tokens, logprobs, margins, topk_tokens


def sample_from_list(topk_tokens, topk_scores, temperature, seed, draw) -> Sample:
    """The draw of top-k sampling from given per-row lists (tokens and float32
    scores, best first): weights w_i = exp((s_i - s_1) / temperature) and
    their running sums in rank order in float32, one Philox uniform per row
    (counter (row, draw)), the first rank whose running sum exceeds u * S
    (the last if none)."""
    toks_in = np.asarray(topk_tokens)
    sc = np.asarray(topk_scores, dtype=np.float32)
    R, k = sc.shape
    toks = np.empty(R, np.int32)
    lps = np.empty(R, np.float64)
    margins = np.empty(R, np.float64)
    tau = np.float32(temperature)
    for r in range(R):
        s = sc[r]
        w = [np.float32(np.exp(np.float32(np.float32(s[i] - s[0]) / tau))) for i in range(k)]
        c, acc = [], np.float32(0.0)
        for wi in w:
            acc = np.float32(acc + wi)
            c.append(acc)
        S = acc
        u = sample_uniform(seed, r, draw)
        t = np.float32(u * S)
        i = next((j for j in range(k) if t < c[j]), k - 1)
        toks[r] = toks_in[r, i]
        lps[r] = float(np.log(np.float64(w[i]) / np.float64(S)))
        margins[r] = min(abs(float(t) - float(cj)) for cj in c) / float(S)
    return Sample(toks, lps, margins, toks_in)


def sample(logits, dtype, k, temperature, seed, draw) -> Sample:
    """Top-k sampling by its definition: every row's exact top-k (the oracle's
    full log-softmax and full sort, with one beam and a zero running score),
    then the draw of sample_from_list on those lists."""
    x = _logits(logits, dtype)
    R, V = x.shape
    res = step(x.reshape(R, 1, V), dtype, np.zeros((R, 1), np.float32), None, k, eos_id=0)
    return sample_from_list(res.token_ids, res.scores, temperature, seed, draw)
