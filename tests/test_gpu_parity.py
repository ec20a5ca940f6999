"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Indices must match bit for bit except at near-ties; scores within 1e-5
relative for float32 logits and 2e-3 for float16/bfloat16 (floor 1), the rule
in tests/compare.py. Workloads are the five seeded configurations at full size
plus edge cases: ragged and misaligned rows, tiny vocabularies, k = V, k = 1,
non-power-of-two k, k = 64, every beam finished, exact ties, -inf logits,
forced per-piece overflow, every register-tile variant, the caller-workspace
entry point, and bit-exact repeatability.
"""
import numpy as np
import pytest
import torch

import oracle
from beam_search_top_amd import rtopk, synth
from compare import compare, exact_index_problems
from gpu_util import DEV, misaligned_copy, run, to_device

pytestmark = pytest.mark.gpu


def check(s, got, nthreads=8):
    """The parity rule, then exact (beam, token) wherever the oracle's fp64
    score is more than 1e-5 * max(|s|, 1) away from its neighbours."""
    ref = oracle.step_of(s, nthreads=nthreads)
    problems = compare(s, got[0], got[1], got[2], ref)
    assert not problems, f"{s.name} seed={s.seed}:\n" + "\n".join(problems)
    ref_next = oracle.step(s.logits, s.dtype, s.alive, s.finished, s.k + 1, s.eos_id, nthreads)
    exact, swaps = exact_index_problems(s, got[0], got[1], ref, ref_next)
    assert not exact, f"{s.name} seed={s.seed}:\n" + "\n".join(exact[:10])
    print(f"[parity] {s.name} seed={s.seed}: near-tie swaps accepted {swaps}", flush=True)
    return ref


@pytest.mark.parametrize("name", ["tiny", "c32k", "spiked40k", "b128"])
@pytest.mark.parametrize("seed_off", [0, 1, 2])
def test_configs(name, seed_off):
    s = synth.make_step(name, synth.default_seed(name) + 100 * seed_off)
    print(f"[parity] {name} seed={s.seed}", flush=True)
    check(s, run(s))


def test_config_mixed250k():
    s = synth.make_step("mixed250k")
    print(f"[parity] mixed250k seed={s.seed}", flush=True)
    check(s, run(s), nthreads=16)


def test_tiny_against_exact_indices():
    s = synth.make_step("tiny")
    got = run(s)
    ref = oracle.step_of(s)
    assert np.array_equal(got[0], ref.beam_ids) and np.array_equal(got[1], ref.token_ids)


EDGE = [
    # B, beam, k, V, dtype, kwargs
    (3, 4, 4, 1001, synth.F16, {}),                  # ragged rows: V*2 bytes not a multiple of 16
    (2, 3, 3, 37, synth.F32, {}),                    # tiny ragged vocabulary, k = 3 (8 groups... 4)
    (2, 2, 2, 3, synth.BF16, {}),                    # V < vector width
    (1, 1, 4, 4, synth.F32, {}),                     # k = V = beam*V
    (5, 1, 7, 700, synth.F16, {}),                   # beam = 1, odd k
    (1, 6, 1, 5000, synth.BF16, {}),                 # k = 1, B = 1
    (2, 16, 64, 5000, synth.F16, {}),                # k = 64 (max), ngroups 64
    (3, 5, 5, 2999, synth.F32, {"n_finished": 4}),   # k = 5 -> 8 groups, finished beams
    (1, 32, 8, 250000, synth.BF16, {}),              # 1312 pieces per batch element, 10496 published slots
    (2, 8, 8, 250000, synth.BF16, {"dist": "uniform", "sigma": 0.001}),  # ~70 ties per piece
    (4, 3, 3, 40000, synth.BF16, {"dist": "gumbel"}),
    (2, 4, 4, 40000, synth.F16, {"dist": "int"}),    # small integers: heavy exact ties
    (2, 4, 4, 40000, synth.F16, {"dist": "uniform", "sigma": 60000.0}),  # large finite magnitudes
    (2, 8, 8, 100000, synth.F32, {"dist": "uniform", "sigma": 0.001}),
    (1, 2, 2, 8, synth.F32, {"n_finished": 1}),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}x{c[3]}k{c[2]}d{c[4]}" for c in EDGE])
def test_edge_shapes(case):
    B, beam, k, V, dt, kw = case
    s = synth.make_custom(B, beam, k, V, dt, seed=4242 + V + k, **kw)
    s.eos_id = min(2, V - 1)
    print(f"[parity] {s.name}", flush=True)
    check(s, run(s))


def test_all_finished_pads():
    s = synth.make_custom(3, 2, 5, 50, synth.F16, seed=7, n_finished=6)
    got = run(s)
    ref = check(s, got)
    assert (got[0][:, 2:] == -1).all() and (got[1][:, 2:] == -1).all()
    assert np.isneginf(got[2][:, 2:]).all()
    assert np.array_equal(got[2][:, :2], ref.scores[:, :2])  # frozen scores, bit-exact


def test_constant_rows_tie_break_bf16():
    s = synth.make_custom(4, 8, 8, 250000, synth.BF16, seed=3, const=1.0)
    s.alive[:] = -2.5  # all beams tie too: pure flat-index order
    got = run(s)
    check(s, got)
    assert (got[0] == 0).all() and (got[1] == np.arange(8)[None, :]).all()


def test_constant_rows_tie_break_f16_sorted_in_lds():
    # every piece is all ties (its exact top-k comes from argmax rounds) and all
    # 8 * 4 * 4 published candidates tie in score: more survivors than lanes
    s = synth.make_custom(2, 4, 4, 40000, synth.F16, seed=13, const=0.5)
    s.alive[:] = -1.0
    got = run(s)
    check(s, got)
    assert (got[0] == 0).all() and (got[1] == np.arange(4)[None, :]).all()


def test_duplicate_beams_tie_by_flat_index():
    s = synth.make_custom(3, 4, 4, 40000, synth.F16, seed=12, sigma=3.0)
    s.logits[:, 2] = s.logits[:, 0]
    s.alive[:, 2] = s.alive[:, 0]
    got = run(s)
    check(s, got)
    # identical rows must get identical scores on the GPU (deterministic lse)
    for b in range(3):
        for p in range(4):
            if got[0][b, p] == 2:
                q = np.where((got[0][b] == 0) & (got[1][b] == got[1][b, p]))[0]
                if len(q):
                    assert got[2][b, q[0]] == got[2][b, p]


def test_finished_rows_are_never_used():
    # a finished row's logits may be loaded but must not reach any result:
    # fill them with NaN and +inf (outside the contract for alive rows)
    s = synth.make_custom(8, 4, 4, 40000, synth.F16, seed=31, sigma=3.0, n_finished=9)
    fin = s.finished.astype(bool)
    garbage = np.array([np.nan, np.inf], np.float16)
    s.logits[fin] = garbage[np.arange(s.V) % 2][None, :]
    check(s, run(s))


def test_neg_inf_logits():
    s = synth.make_custom(2, 4, 4, 3000, synth.F32, seed=99, sigma=2.0)
    rng = np.random.default_rng(5)
    mask = rng.random(s.logits.shape) < 0.5
    s.logits[mask] = -np.inf
    check(s, run(s))


@pytest.mark.parametrize("offset", [1, 3, 5, 7])
def test_misaligned_base_pointer(offset):
    s = synth.make_custom(4, 4, 4, 4096, synth.F16, seed=21 + offset, sigma=3.0, n_finished=2)
    x = misaligned_copy(s, offset)
    a = torch.from_numpy(s.alive).to(DEV)
    f = torch.from_numpy(s.finished).to(DEV)
    assert x.data_ptr() % 16 != 0
    out = rtopk.beam_step(x, a, f, k=s.k, eos_id=s.eos_id)
    torch.cuda.synchronize()
    check(s, [o.cpu().numpy() for o in out])


def test_forced_overflow_path_is_exact():
    # chunk limit 1 (raised to k): every piece with more than k candidates emits its exact top-k
    cases = [synth.make_step("b128"), synth.make_custom(2, 8, 8, 250000, synth.BF16, seed=5, const=1.0),
             synth.make_custom(3, 4, 4, 40000, synth.F16, seed=6, dist="int")]
    assert rtopk.rtopk_set_override(0, 1) == 0
    try:
        for s in cases:
            print(f"[parity overflow] {s.name}", flush=True)
            check(s, run(s))
    finally:
        rtopk.rtopk_set_override(0, 0)


def test_row_local_and_published_paths_agree():
    # shapes whose pieces per row divide the workgroup run row-local by
    # default; the same shapes through the per-piece publication path
    cases = [synth.make_step("b128"), synth.make_step("c32k"), synth.make_step("tiny"),
             synth.make_custom(2, 16, 64, 5000, synth.F16, seed=77),
             synth.make_custom(3, 5, 5, 2999, synth.F32, seed=78, n_finished=4),
             synth.make_custom(5, 1, 7, 700, synth.F16, seed=79)]
    for s in cases:
        st, p = rtopk.rtopk_plan(None, s.B, s.beam, s.V, s.k, s.dtype)
        assert st == 0 and p.row_local == 1, s.name
    got_rl = [run(s) for s in cases]
    assert rtopk.rtopk_set_row_local(0) == 0
    try:
        for s, g in zip(cases, got_rl):
            print(f"[parity published] {s.name}", flush=True)
            ref = check(s, run(s))
            check(s, g)
            del ref
    finally:
        rtopk.rtopk_set_row_local(1)


def test_split_and_in_kernel_selection_agree():
    # per-piece publication in rounds (more pieces than the GPU holds at once):
    # the per-batch selection runs as a second launch by default, inside the
    # step kernel with the switch off; both must match the oracle and each other
    cases = [synth.make_step("mixed250k"),
             synth.make_custom(64, 8, 8, 60000, synth.BF16, seed=91, n_finished=9),
             synth.make_custom(40, 6, 5, 70000, synth.F32, seed=92, n_finished=4)]
    for s in cases:
        st, p = rtopk.rtopk_plan(None, s.B, s.beam, s.V, s.k, s.dtype)
        assert st == 0 and p.row_local == 0 and s.B * s.beam * p.chunks > 4096, s.name
    for s in cases:
        print(f"[parity split] {s.name}", flush=True)
        got_split = run(s)
        check(s, got_split, nthreads=16)
        assert rtopk.rtopk_set_split(0) == 0
        try:
            got_in = run(s)
        finally:
            rtopk.rtopk_set_split(1)
        for a, b in zip(got_split, got_in):
            assert np.array_equal(a, b), s.name


@pytest.mark.parametrize("nv", [1, 2, 3, 4, 6, 8, 10, 12])
def test_every_tile_variant(nv):
    cases = [synth.make_custom(4, 4, 4, 40000, synth.F16, seed=300 + nv, sigma=3.0, n_finished=1),
             synth.make_custom(2, 4, 4, 32000, synth.F32, seed=400 + nv, sigma=2.0),
             synth.make_custom(2, 8, 8, 50000, synth.BF16, seed=500 + nv, dist="gumbel"),
             synth.make_custom(2, 3, 3, 20001, synth.F16, seed=600 + nv, sigma=3.0)]
    assert rtopk.rtopk_set_override(nv, 0) == 0
    try:
        for s in cases:
            check(s, run(s))
    finally:
        rtopk.rtopk_set_override(0, 0)


def test_workspace_entry_point_matches_and_reuses():
    s1 = synth.make_step("b128")
    s2 = synth.make_custom(5, 4, 4, 40000, synth.F16, seed=77, n_finished=2)
    nbytes = max(rtopk.rtopk_workspace_bytes(s.B, s.beam, s.V, s.k, s.dtype) for s in (s1, s2))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for s in (s1, s2, s1):
        x, a, f = to_device(s)
        plain = rtopk.beam_step(x, a, f, k=s.k)
        with_ws = rtopk.beam_step(x, a, f, k=s.k, workspace=ws)
        torch.cuda.synchronize()
        for p, w in zip(plain, with_ws):
            assert torch.equal(p, w)
        check(s, [o.cpu().numpy() for o in with_ws])


def test_repeatable_bit_for_bit():
    s = synth.make_step("b128")
    x, a, f = to_device(s)
    first = [o.clone() for o in rtopk.beam_step(x, a, f, k=s.k)]
    for _ in range(20):
        again = rtopk.beam_step(x, a, f, k=s.k)
        for p, q in zip(first, again):
            assert torch.equal(p, q)
    torch.cuda.synchronize()


def test_streams_have_separate_workspaces():
    s = synth.make_step("b128")
    x, a, f = to_device(s)
    ref = [o.clone() for o in rtopk.beam_step(x, a, f, k=s.k)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = []
    for st in streams:
        with torch.cuda.stream(st):
            outs.append(rtopk.beam_step(x, a, f, k=s.k))
    torch.cuda.synchronize()
    for o in outs:
        for p, q in zip(ref, o):
            assert torch.equal(p, q)


def test_library_workspace_survives_shape_changes():
    # Regression: the library-owned workspace is reused across shapes on one
    # stream; a larger call must not find stale data where its counters live.
    names = ["tiny", "c32k", "spiked40k", "b128", "tiny", "b128", "c32k"]
    for n in names:
        s = synth.make_step(n)
        check(s, run(s))


def test_caller_workspace_tickets_return_to_zero():
    # Only the fixed region (arrival counters, status words, mailbox) must be
    # zero between calls; calls of different shapes then share one caller
    # workspace (row-local and per-piece shapes alternate here).
    s_small = synth.make_custom(3, 4, 4, 40000, synth.F16, seed=31, n_finished=1)
    s_big = synth.make_step("b128")
    nbytes = rtopk.rtopk_workspace_bytes(s_big.B, s_big.beam, s_big.V, s_big.k, s_big.dtype)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    s_pub = synth.make_custom(2, 3, 3, 20001, synth.F16, seed=32, n_finished=1)
    st, p = rtopk.rtopk_plan(None, s_pub.B, s_pub.beam, s_pub.V, s_pub.k, s_pub.dtype)
    assert st == 0 and p.row_local == 0
    nbytes = max(nbytes, rtopk.rtopk_workspace_bytes(s_pub.B, s_pub.beam, s_pub.V, s_pub.k, s_pub.dtype))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for s in (s_small, s_big, s_pub, s_small, s_big, s_pub, s_big):
        x, a, f = to_device(s)
        out = rtopk.beam_step(x, a, f, k=s.k, workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:rtopk.RTOPK_WS_FIXED_BYTES])) == 0
        check(s, [o.cpu().numpy() for o in out])


def test_wait_give_up_is_reported_and_cleared():
    # The merge of a batch element whose rows span workgroups waits for the
    # others' lists with a bounded poll. A bound of 0 makes every such merge
    # give up at once (no kernel waits or faults): its outputs are padding,
    # rtopk_check reports RTOPK_ETIMEOUT and clears the workspace, and the
    # next call is exact again.
    s = synth.make_step("b128")
    st, p = rtopk.rtopk_plan(None, s.B, s.beam, s.V, s.k, s.dtype)
    assert st == 0 and p.row_local == 1 and p.pieces_per_group < s.beam * p.chunks  # rows span workgroups
    x, a, f = to_device(s)
    stream = torch.cuda.current_stream().cuda_stream
    for use_ws in (False, True):
        ws = None
        if use_ws:
            ws = torch.zeros(rtopk.rtopk_workspace_bytes(s.B, s.beam, s.V, s.k, s.dtype), dtype=torch.uint8,
                             device=DEV)
        wsp = None if ws is None else ws.data_ptr()
        rtopk.beam_step(x, a, f, k=s.k, workspace=ws)
        assert rtopk.rtopk_check(wsp, stream) == rtopk.RTOPK_OK
        assert rtopk.rtopk_set_spin_limit(0) == 0
        try:
            out = rtopk.beam_step(x, a, f, k=s.k, workspace=ws)
            torch.cuda.synchronize()
        finally:
            rtopk.rtopk_set_spin_limit(rtopk.RTOPK_DEFAULT_SPIN_LIMIT)
        assert (out[0] == -1).all() and (out[1] == -1).all() and torch.isneginf(out[2]).all()
        assert rtopk.rtopk_check(wsp, stream) == rtopk.RTOPK_ETIMEOUT
        assert "gave up" in rtopk.rtopk_last_error()
        assert rtopk.rtopk_check(wsp, stream) == rtopk.RTOPK_OK  # cleared
        if ws is not None:
            assert int(torch.count_nonzero(ws[:rtopk.RTOPK_WS_FIXED_BYTES])) == 0
        out = rtopk.beam_step(x, a, f, k=s.k, workspace=ws)
        torch.cuda.synchronize()
        check(s, [o.cpu().numpy() for o in out])
        assert rtopk.rtopk_check(wsp, stream) == rtopk.RTOPK_OK


def test_candidate_scoring_exactly_at_the_bound():
    # Regression: in b=105 of this seed the 4th-best candidate's logit equals
    # its piece's threshold, so its score equals the batch bound exactly; the
    # bound and the score must be rounded the same way for it to survive.
    s = synth.make_step("b128", synth.default_seed("b128") + 100)
    got = run(s)
    check(s, got)
    ref = oracle.step_of(s)
    assert got[1][105, 3] == ref.token_ids[105, 3]


@pytest.mark.parametrize("B,beam,k,V,dt,dist", [
    (32, 1, 64, 50000, synth.BF16, "gumbel"), (16, 2, 64, 40000, synth.F16, "int"),
    (8, 1, 48, 100000, synth.BF16, "gumbel"),
])
def test_more_survivors_than_lds_keys(B, beam, k, V, dt, dist):
    # regression: a batch element whose survivors outnumber the LDS sort keys
    # (512) but not the workgroup's threads must take the argmax rounds, not
    # rank the first 512 and read past them
    s = synth.make_custom(B, beam, k, V, dt, seed=B * 31 + k, dist=dist, sigma=1.0)
    st, p = rtopk.rtopk_plan(None, s.B, s.beam, s.V, s.k, s.dtype)
    assert st == 0
    print(f"[parity] {s.name} row_local={p.row_local} sort_keys={p.sort_keys} threads={p.pieces_per_group * 64}",
          flush=True)
    check(s, run(s))


@pytest.mark.parametrize("B,beam,k,V,dt,ties", [
    (2, 4, 8, 40000, synth.F16, 768),      # ~96 tied top logits per piece, row-local path
    (2, 4, 64, 40000, synth.F32, 1536),    # k = 64 drawn from ~96 ties per piece
    (2, 8, 8, 250000, synth.BF16, 5952),   # per-piece publication path
])
def test_more_hits_than_lanes(B, beam, k, V, dt, ties):
    # pieces with 65..128 hits stage two keys per lane and rank both halves
    s = synth.make_custom(B, beam, k, V, dt, seed=ties + k, top_ties=ties)
    print(f"[parity] {s.name}", flush=True)
    check(s, run(s))


@pytest.mark.parametrize("B,beam,k,V,dt,kw", [
    (2, 8, 8, 250000, synth.BF16, dict(const=1.0)),                  # every slot survives: 3968 keys
    (3, 8, 8, 250000, synth.BF16, dict(const=1.0, n_finished=2)),    # ... and finished beams offer their end token
    (2, 8, 4, 250000, synth.F16, dict(dist="int")),                  # heavy ties across beams
    (2, 8, 16, 250000, synth.BF16, dict(const=0.5)),                 # 7936 slots
])
def test_survivors_past_lds_keys_small_k(B, beam, k, V, dt, kw):
    # the per-batch selection with more survivors than its LDS keys and a
    # small k: the argmax rounds over every published slot, with ties
    s = synth.make_custom(B, beam, k, V, dt, seed=k + beam, **kw)
    st, p = rtopk.rtopk_plan(None, s.B, s.beam, s.V, s.k, s.dtype)
    assert st == 0 and not p.row_local
    print(f"[parity] {s.name} slots/batch={beam * p.chunks * k} sort_keys={p.sort_keys} "
          f"threads={p.pieces_per_group * 64}", flush=True)
    check(s, run(s))


@pytest.mark.parametrize("B,beam,k,V,dt,nfin", [
    (16, 4, 12, 40000, synth.F16, 3), (8, 8, 24, 40000, synth.BF16, 4), (6, 2, 9, 40000, synth.F32, 2),
    (12, 4, 15, 20000, synth.F16, 5), (256, 2, 12, 40000, synth.F16, 7),
])
def test_row_local_large_k_with_finished_beams(B, beam, k, V, dt, nfin):
    # 8 < k < 16: row-local workgroups may hold rows of several batch elements
    # (the one-batch-element rule applies from k = 16), so the k > 8 selection
    # and its per-batch loop run over several of them; finished beams offer
    # their end token there too
    s = synth.make_custom(B, beam, k, V, dt, seed=900 + k, sigma=3.0, n_finished=nfin)
    st, p = rtopk.rtopk_plan(None, B, beam, V, k, dt)
    assert st == 0 and p.row_local == 1, (s.name, p.as_dict())
    print(f"[parity row-local k>8] {s.name} waves {p.pieces_per_group} chunks {p.chunks}", flush=True)
    check(s, run(s))
