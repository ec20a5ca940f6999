"""The step fused into the LM head (rtopk_lmhead_step, through the C ABI)
against the oracle: the float64 GEMM of the same bfloat16 hidden states and
weights, then the float64 step. Scores within 2e-3 * max(|s|, 1) (bfloat16
inputs); indices bit-exact wherever the oracle's float64 score is more than
1e-4 * max(|s|, 1) from its neighbours (the GPU's logits carry float32
accumulation, about 1e-4 at H = 1024), near-ties allowed by the parity rule
elsewhere. Small and ragged shapes are checked whole; the 128 x 4 x 1024 x
40000 shape on a sample of batch elements (the oracle's GEMM is slow)."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from beam_search_top_amd import rtopk, synth
from compare import compare, exact_index_problems
from libutil import ensure_built

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, beam, H, V, seed, n_finished=0, sigma=3.0):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.normal(0, 1, (B * beam, H)).astype(np.float32))
    w = synth.f32_to_bf16_bits(rng.normal(0, sigma / np.sqrt(H), (V, H)).astype(np.float32))
    alive = rng.uniform(-30, 0, (B, beam)).astype(np.float32)
    fin = np.zeros(B * beam, np.uint8)
    if n_finished:
        fin[rng.choice(B * beam, n_finished, replace=False)] = 1
    return x, w, alive, fin.reshape(B, beam)


def _run(x, w, alive, fin, k, eos):
    ensure_built()
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(DEV)
    out = rtopk.lmhead_step(xt, wt, torch.from_numpy(alive).to(DEV), torch.from_numpy(fin).to(DEV), k=k,
                            eos_id=eos)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _check(x, w, alive, fin, beam, k, eos, got, rows_of=None):
    """rows_of: the batch elements to check (all when None)."""
    B = alive.shape[0]
    bs = list(range(B)) if rows_of is None else list(rows_of)
    rows = np.concatenate([np.arange(b * beam, (b + 1) * beam) for b in bs])
    logits = oracle.lmhead_logits(x[rows], w)
    V = w.shape[0]
    sub = SimpleNamespace(B=len(bs), beam=beam, V=V, k=k, dtype=oracle.F64, logits=logits.reshape(len(bs), beam, V),
                          alive=alive[bs], finished=fin[bs], eos_id=eos)
    ref = oracle.step(sub.logits, oracle.F64, sub.alive, sub.finished, k, eos, nthreads=8)
    g = [o[bs] for o in got]
    problems = compare(sub, g[0], g[1], g[2], ref, rtol=2e-3)
    assert not problems, "\n".join(problems[:10])
    nxt = oracle.step(sub.logits, oracle.F64, sub.alive, sub.finished, k + 1, eos, nthreads=8)
    exact, swaps = exact_index_problems(sub, g[0], g[1], ref, nxt, rel=1e-4)
    assert not exact, "\n".join(exact[:10])
    return swaps


@pytest.mark.parametrize("B,beam,H,V,k,nfin", [
    (2, 2, 64, 300, 2, 0),       # one 320-wide vocabulary tile, ragged inside a thread's 40 columns
    (2, 2, 64, 700, 2, 0),       # three vocabulary tiles, the last 60 wide (whole threads past V)
    (3, 4, 128, 1000, 4, 2),     # 12 rows of one 256-row tile, finished beams
    (5, 1, 64, 7, 1, 0),         # V < 40: part of one thread's columns, k = 1
    (2, 8, 192, 2000, 8, 3),     # k = 8 (8 groups), beam = 8
    (4, 4, 64, 640, 5, 1),       # k = 5: the 5th largest of 8 group maxima; two whole tiles
    (65, 4, 64, 700, 4, 5),      # 260 rows: two row tiles, the second with 4 rows
    (33, 4, 256, 4100, 4, 6),    # 132 rows, 13 vocabulary tiles
    (1, 3, 64, 128, 3, 3),       # every beam finished
])
def test_lmhead_matches_oracle(B, beam, H, V, k, nfin):
    x, w, alive, fin = _inputs(B, beam, H, V, seed=B * 1000 + V + k, n_finished=nfin)
    eos = min(2, V - 1)
    print(f"[lmhead] B={B} beam={beam} H={H} V={V} k={k} finished={nfin}", flush=True)
    got = _run(x, w, alive, fin, k, eos)
    swaps = _check(x, w, alive, fin, beam, k, eos, got)
    print(f"[lmhead] near-tie swaps accepted {swaps}", flush=True)


def test_lmhead_full_size_sampled():
    B, beam, H, V, k = 128, 4, 1024, 40000, 4
    x, w, alive, fin = _inputs(B, beam, H, V, seed=2026, n_finished=26)
    got = _run(x, w, alive, fin, k, 2)
    sample = [0, 1, 37, 64, 101, 126, 127]
    print(f"[lmhead] full size, batch elements {sample}", flush=True)
    swaps = _check(x, w, alive, fin, beam, k, 2, got, rows_of=sample)
    print(f"[lmhead] near-tie swaps accepted {swaps}", flush=True)
    # every batch element: valid, distinct, ordered (the oracle is sampled)
    for b in range(B):
        pairs = set(zip(got[0][b].tolist(), got[1][b].tolist()))
        assert len(pairs) == k and all(0 <= j < beam and 0 <= t < V for j, t in pairs)
        assert all(got[2][b][i] >= got[2][b][i + 1] for i in range(k - 1))


def test_lmhead_rejects_before_launch():
    ensure_built()
    p = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    a = torch.zeros(4, dtype=torch.float32, device=DEV)
    o = torch.zeros(64, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    args = lambda B, beam, H, V, k, eos: rtopk.rtopk_lmhead_step(p.data_ptr(), p.data_ptr(), a.data_ptr(), None, B, beam,
                                                                 H, V, k, eos, o.data_ptr(), o.data_ptr(),
                                                                 o.data_ptr(), s)
    assert args(1, 2, 100, 300, 2, 0) == rtopk.RTOPK_ENOTSUP   # H not a multiple of 64
    assert args(1, 2, 64, 300, 9, 0) == rtopk.RTOPK_ENOTSUP    # k > 8
    assert args(1, 2, 64, 300, 2, 300) == rtopk.RTOPK_EINVAL   # eos outside [0, V)
    assert args(1, 1, 64, 1, 2, 0) == rtopk.RTOPK_EINVAL       # k > beam * V
    torch.cuda.synchronize()
    assert (o == 0).all()
