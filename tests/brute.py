"""Brute-force decode-step selection for tiny inputs, independent of the oracle.

Every (beam, token) pair is enumerated; log-sum-exp is taken in 50-digit
decimal arithmetic straight from its definition, log(sum_t exp(x_t)), with no
max shift; pairs are ordered with Python's ``sorted`` by (score desc, flat
asc). Logits come in as float64 (exact conversions made by numpy), so this
shares nothing with the C oracle except the problem statement.
"""
from decimal import Decimal, localcontext

import numpy as np


def brute_topk(x64, alive, finished, k, eos_id):
    """x64 [B, beam, V] float64; returns (beam_ids, token_ids, scores as Decimal lists, lse)."""
    B, beam, V = x64.shape
    out_b = np.full((B, k), -1, np.int64)
    out_t = np.full((B, k), -1, np.int64)
    out_s = [[None] * k for _ in range(B)]
    lse = [[None] * beam for _ in range(B)]
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            entries = []
            for j in range(beam):
                a = Decimal(float(alive[b, j]))
                if finished is not None and finished[b, j]:
                    entries.append((a, j * V + eos_id))
                    continue
                xs = [Decimal(float(v)) for v in x64[b, j]]
                z = sum((xv.exp() for xv in xs), Decimal(0)).ln()
                lse[b][j] = z
                entries.extend((a + (xv - z), j * V + t) for t, xv in enumerate(xs))
            ranked = sorted(entries, key=lambda e: (-e[0], e[1]))
            for p, (s, flat) in enumerate(ranked[:k]):
                out_b[b, p], out_t[b, p], out_s[b][p] = flat // V, flat % V, s
    return out_b, out_t, out_s, lse


def brute_scores(x64, alive, finished, eos_id):
    """Every pair's score by the definition, in 50-digit decimals:
    {(b, j, t): Decimal} for the candidates of each batch element (every token
    of an alive beam; only (j, eos_id) of a finished beam, at its running
    score). Pairs missing from the dict are not candidates."""
    B, beam, V = x64.shape
    out = {}
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            for j in range(beam):
                a = Decimal(float(alive[b, j]))
                if finished is not None and finished[b, j]:
                    out[(b, j, eos_id)] = a
                    continue
                xs = [Decimal(float(v)) for v in x64[b, j]]
                z = sum((xv.exp() for xv in xs), Decimal(0)).ln()
                for t, xv in enumerate(xs):
                    out[(b, j, t)] = a + (xv - z)
    return out
