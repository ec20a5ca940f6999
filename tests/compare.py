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


EXACT_REL = 1e-5  # fp64 score gap above which a position's pair is decidable exactly


def exact_index_problems(step, got_beam, got_token, ref, ref_next, rel=EXACT_REL):
    """Positions whose pair must match the oracle's exactly: those where the
    oracle's fp64 score is more than rel * max(|s|, 1) away from both
    neighbours (positions p - 1, p + 1, and for the last position the
    (k+1)-th candidate, taken from ref_next = the oracle run with k + 1).
    Returns (problems, accepted_swaps): accepted_swaps counts positions where
    the pair differs from the oracle's but lies inside that window."""
    B, k = step.B, step.k
    got_beam = np.asarray(got_beam).reshape(B, k)
    got_token = np.asarray(got_token).reshape(B, k)
    s = np.asarray(ref_next.scores64).reshape(B, k + 1)
    assert np.array_equal(np.asarray(ref_next.beam_ids)[:, :k], ref.beam_ids)
    assert np.array_equal(np.asarray(ref_next.token_ids)[:, :k], ref.token_ids)
    problems, swaps = [], 0
    for b in range(B):
        for p in range(k):
            if ref.beam_ids[b, p] < 0:
                continue
            sp = s[b, p]
            w = rel * max(abs(sp), 1.0)
            near = (p > 0 and s[b, p - 1] - sp <= w) or (sp - s[b, p + 1] <= w)
            same = (int(got_beam[b, p]), int(got_token[b, p])) == (int(ref.beam_ids[b, p]), int(ref.token_ids[b, p]))
            if same:
                continue
            if near:
                swaps += 1
            else:
                problems.append(f"b={b} p={p}: got ({got_beam[b, p]},{got_token[b, p]}), oracle "
                                f"({ref.beam_ids[b, p]},{ref.token_ids[b, p]}) with fp64 gaps above {w:.3g}")
    return problems, swaps
