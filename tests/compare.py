"""Tie-aware parity rule between a decode step's output and the CPU oracle's.

Scores: |got - oracle| <= rtol * max(|oracle|, 1), rtol 1e-5 for float32 logits
and 2e-3 for float16 / bfloat16 logits. Indices: equal at every position,
except that a differing pair is accepted when the oracle's own score of that
pair is within the same tolerance of the oracle's score at that position (a
near-tie). In every case the returned pairs must be distinct, valid
candidates, and ordered by (score desc, flat index asc) in the returned
scores.
"""
import math

import numpy as np

import oracle

RTOL = {0: 1e-5, 1: 2e-3, 2: 2e-3}


def tol_of(dtype, ref):
    return RTOL[dtype] * max(abs(ref), 1.0)


def compare(step, got_beam, got_token, got_score, ref, rtol=None, max_report=10):
    """Return a list of human-readable problems (empty when the outputs agree)."""
    B, beam, V, k = step.B, step.beam, step.V, step.k
    got_beam = np.asarray(got_beam).reshape(B, k)
    got_token = np.asarray(got_token).reshape(B, k)
    got_score = np.asarray(got_score, dtype=np.float32).reshape(B, k)
    problems = []
    r = RTOL[step.dtype] if rtol is None else rtol

    def tol(x):
        return r * max(abs(x), 1.0)

    for b in range(B):
        seen = set()
        prev = None
        for p in range(k):
            gb, gt, gs = int(got_beam[b, p]), int(got_token[b, p]), float(got_score[b, p])
            ob, ot, os64 = int(ref.beam_ids[b, p]), int(ref.token_ids[b, p]), float(ref.scores64[b, p])
            where = f"b={b} p={p} got=({gb},{gt},{gs!r}) oracle=({ob},{ot},{os64!r})"
            if ob < 0:  # oracle pads: the output must pad too
                if not (gb == -1 and gt == -1 and gs == -math.inf):
                    problems.append("expected padding at " + where)
                continue
            if gb < 0 or gt < 0:
                problems.append("unexpected padding at " + where)
                continue
            if (gb, gt) in seen:
                problems.append("duplicate pair at " + where)
            seen.add((gb, gt))
            if not (abs(gs - os64) <= tol(os64)):
                problems.append(f"score off by {gs - os64:.3g} (tol {tol(os64):.3g}) at " + where)
            if (gb, gt) != (ob, ot):
                s_of = oracle.score_of(step.logits, step.dtype, step.alive, step.finished, ref.lse,
                                       step.eos_id, b, gb, gt)
                if not (abs(s_of - os64) <= tol(os64)):
                    problems.append(f"index mismatch, not a near-tie (oracle score of got pair {s_of!r}) at "
                                    + where)
            key = (-gs, gb * V + gt)
            if prev is not None and key < prev:
                problems.append("output not ordered by (score desc, flat asc) at " + where)
            prev = key
        if len(problems) >= max_report:
            break
    return problems
