"""Seeded synthetic inputs for one beam-search decode step.

This module draws logits, running (alive) scores and finished masks, and
nothing else: it holds none of the selection arithmetic, so both the HIP path
and the CPU oracle can be fed from it without sharing any of the method.

Workload shapes follow the LightSeq inference article's decoding passage:
a [batch_size, beam_size, vocab_size] logit matrix, a vocabulary in the tens
of thousands, logits that the article takes to be roughly normal, and top-4
selection; the 40k vocabulary is the one of the LightSeq training article's
benchmark set-up (WMT14 en-de). No dataset or trained model is involved.

Recipes (numpy PCG64, ``default_rng(seed)``; draws in float64/float32, then
round-to-nearest-even into the logit dtype):

* ``tiny``      B=2,   beam=2, k=2, V=8,      fp32 N(0,1),  alive U(-5,0)
* ``c32k``      B=8,   beam=4, k=4, V=32000,  fp32 N(0,2),  alive U(-20,0),
                exactly 1 of 32 beams finished
* ``spiked40k`` B=32,  beam=4, k=4, V=40000,  fp16 N(0,3) with 8 distinct
                positions per beam set to exactly 10.0, alive U(-30,0)
* ``b128``      B=128, beam=4, k=4, V=40000,  fp16 N(0,3), alive U(-30,0),
                exactly round(0.05*512)=26 beams finished
* ``mixed250k`` B=64,  beam=8, k=8, V=250000, bf16; a seeded permutation
                gives 256 N(0,1) beams, 128 near-flat beams
                (U(-1e-3, 1e-3)) and 128 Gumbel(0,1) beams; alive U(-50,0)

The second argument of N(mu, sigma) is the standard deviation. Finished rows
still hold random logits; a correct step never uses them.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}
EOS_ID = 2


@dataclasses.dataclass
class Step:
    """One decode step's inputs as host arrays.

    logits: [B, beam, V]; float32 for F32, float16 for F16, uint16 bit
    patterns for BF16. alive: [B, beam] float32. finished: [B, beam] uint8.
    """
    name: str
    B: int
    beam: int
    k: int
    V: int
    dtype: int
    logits: np.ndarray
    alive: np.ndarray
    finished: np.ndarray
    eos_id: int = EOS_ID
    seed: int = 0

    @property
    def logit_bytes(self) -> int:
        return self.B * self.beam * self.V * ELEM_BYTES[self.dtype]

    @property
    def n_finished(self) -> int:
        return int(self.finished.sum())


CONFIGS = {
    "tiny": dict(B=2, beam=2, k=2, V=8, dtype=F32),
    "c32k": dict(B=8, beam=4, k=4, V=32000, dtype=F32),
    "spiked40k": dict(B=32, beam=4, k=4, V=40000, dtype=F16),
    "b128": dict(B=128, beam=4, k=4, V=40000, dtype=F16),
    "mixed250k": dict(B=64, beam=8, k=8, V=250000, dtype=BF16),
}
CONFIG_ORDER = ["tiny", "c32k", "spiked40k", "b128", "mixed250k"]


def default_seed(name: str) -> int:
    return 1001 + CONFIG_ORDER.index(name)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def to_dtype(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round a float array into the logit storage type."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x.astype(np.float32).astype(np.float16))
    if dtype == BF16:
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def _finished_mask(rng, B, beam, n_fin):
    mask = np.zeros(B * beam, dtype=np.uint8)
    if n_fin:
        mask[rng.choice(B * beam, size=n_fin, replace=False)] = 1
    return mask.reshape(B, beam)


def make_step(name: str, seed: int | None = None) -> Step:
    """Build one of the named workloads from its recipe (see module docstring)."""
    cfg = CONFIGS[name]
    seed = default_seed(name) if seed is None else seed
    rng = np.random.default_rng(seed)
    B, beam, k, V, dt = cfg["B"], cfg["beam"], cfg["k"], cfg["V"], cfg["dtype"]
    nb = B * beam
    if name == "tiny":
        x = rng.standard_normal((B, beam, V))
        alive = rng.uniform(-5.0, 0.0, (B, beam))
        fin = np.zeros((B, beam), np.uint8)
    elif name == "c32k":
        x = rng.normal(0.0, 2.0, (B, beam, V)).astype(np.float32)
        alive = rng.uniform(-20.0, 0.0, (B, beam))
        fin = _finished_mask(rng, B, beam, 1)
    elif name == "spiked40k":
        x = rng.normal(0.0, 3.0, (nb, V)).astype(np.float32)
        for r in range(nb):
            x[r, rng.choice(V, size=8, replace=False)] = 10.0
        x = x.reshape(B, beam, V)
        alive = rng.uniform(-30.0, 0.0, (B, beam))
        fin = np.zeros((B, beam), np.uint8)
    elif name == "b128":
        x = rng.normal(0.0, 3.0, (B, beam, V)).astype(np.float32)
        alive = rng.uniform(-30.0, 0.0, (B, beam))
        fin = _finished_mask(rng, B, beam, int(round(0.05 * nb)))
    elif name == "mixed250k":
        kinds = rng.permutation(np.repeat(np.arange(3), [nb // 2, nb // 4, nb - nb // 2 - nb // 4]))
        x = np.empty((nb, V), np.float32)
        for r in range(nb):
            if kinds[r] == 0:
                x[r] = rng.standard_normal(V, dtype=np.float32)
            elif kinds[r] == 1:
                x[r] = rng.uniform(-1e-3, 1e-3, V).astype(np.float32)
            else:
                x[r] = rng.gumbel(0.0, 1.0, V).astype(np.float32)
        x = x.reshape(B, beam, V)
        alive = rng.uniform(-50.0, 0.0, (B, beam))
        fin = np.zeros((B, beam), np.uint8)
    else:  # pragma: no cover
        raise KeyError(name)
    return Step(name=name, B=B, beam=beam, k=k, V=V, dtype=dt, logits=to_dtype(x, dt),
                alive=np.ascontiguousarray(alive, dtype=np.float32), finished=fin, seed=seed)


def make_custom(B, beam, k, V, dtype, seed, dist="normal", sigma=1.0, alive_lo=-10.0,
                n_finished=0, const=None, top_ties=0) -> Step:
    """A free-shape step for edge cases: normal / uniform / gumbel / constant rows.

    top_ties > 0 sets that many random positions of every row to one value
    (64.0, exact in every logit type) above all the other draws: the row's
    top logit then repeats top_ties times, ties broken by flat index."""
    rng = np.random.default_rng(seed)
    if const is not None:
        x = np.full((B, beam, V), const, np.float64)
    elif dist == "normal":
        x = rng.normal(0.0, sigma, (B, beam, V))
    elif dist == "uniform":
        x = rng.uniform(-sigma, sigma, (B, beam, V))
    elif dist == "gumbel":
        x = rng.gumbel(0.0, sigma, (B, beam, V))
    elif dist == "int":  # small integers: many exact ties across and within beams
        x = rng.integers(-3, 4, (B, beam, V)).astype(np.float64)
    else:
        raise ValueError(dist)
    if top_ties:
        for row in x.reshape(B * beam, V):
            row[rng.choice(V, size=min(top_ties, V), replace=False)] = 64.0
    alive = rng.uniform(alive_lo, 0.0, (B, beam))
    fin = _finished_mask(rng, B, beam, n_finished)
    tag = f"_ties{top_ties}" if top_ties else ""
    return Step(name=f"custom_{B}x{beam}x{V}_k{k}_{DTYPE_NAMES[dtype]}_{dist}{tag}", B=B, beam=beam, k=k,
                V=V, dtype=dtype, logits=to_dtype(x, dtype),
                alive=np.ascontiguousarray(alive, dtype=np.float32), finished=fin, seed=seed)
