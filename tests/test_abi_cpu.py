"""C-ABI checks that need no GPU: the library loads, exports every function
include/rtopk.h declares, validates arguments before touching HIP, and plans
the decomposition consistently. No call here reaches a kernel launch."""
import ctypes
import math

import pytest

from beam_search_top_amd import rtopk
from libutil import ensure_built

FAKE = 0x7000_0000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_exports_every_declared_function(lib):
    names = rtopk.declared_functions()
    assert set(names) >= {"rtopk_beam_step", "rtopk_beam_step_ws", "rtopk_workspace_bytes",
                          "rtopk_debug_step", "rtopk_plan", "rtopk_set_override",
                          "rtopk_last_error", "rtopk_release"}
    for n in names:
        assert hasattr(lib, n), n
        assert callable(getattr(rtopk, n)), n  # the binding mirrors every name


def _step(**kw):
    a = dict(logits=FAKE, dtype=1, alive=FAKE, fin=None, B=2, beam=4, V=100, k=4, eos=2,
             ob=FAKE, ot=FAKE, os=FAKE)
    a.update(kw)
    return rtopk.rtopk_beam_step(a["logits"], a["dtype"], a["alive"], a["fin"], a["B"], a["beam"], a["V"],
                                 a["k"], a["eos"], a["ob"], a["ot"], a["os"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(logits=None), rtopk.RTOPK_EINVAL, "logits"),
    (dict(alive=None), rtopk.RTOPK_EINVAL, "alive"),
    (dict(ob=None), rtopk.RTOPK_EINVAL, "output"),
    (dict(ot=None), rtopk.RTOPK_EINVAL, "output"),
    (dict(os=None), rtopk.RTOPK_EINVAL, "output"),
    (dict(dtype=3), rtopk.RTOPK_EINVAL, "dtype"),
    (dict(dtype=-1), rtopk.RTOPK_EINVAL, "dtype"),
    (dict(B=0), rtopk.RTOPK_EINVAL, "sizes"),
    (dict(beam=0), rtopk.RTOPK_EINVAL, "sizes"),
    (dict(V=0), rtopk.RTOPK_EINVAL, "sizes"),
    (dict(k=0), rtopk.RTOPK_EINVAL, "sizes"),
    (dict(k=-3), rtopk.RTOPK_EINVAL, "sizes"),
    (dict(beam=2, V=3, k=7), rtopk.RTOPK_EINVAL, "exceeds beam*V"),
    (dict(beam=4, V=2**30), rtopk.RTOPK_EINVAL, "2^31"),
    (dict(eos=100), rtopk.RTOPK_EINVAL, "eos_id"),
    (dict(eos=-1), rtopk.RTOPK_EINVAL, "eos_id"),
    (dict(k=65, beam=8), rtopk.RTOPK_ENOTSUP, "limit"),
    (dict(beam=513, k=4), rtopk.RTOPK_ENOTSUP, "limit"),
    (dict(logits=FAKE + 1), rtopk.RTOPK_EINVAL, "aligned"),
    (dict(logits=FAKE + 2, dtype=0), rtopk.RTOPK_EINVAL, "aligned"),
])
def test_validation_rejects_before_launch(lib, kw, status, msg):
    assert _step(**kw) == status
    assert msg in rtopk.rtopk_last_error()


def test_ws_entry_validation(lib):
    args = (FAKE, 1, FAKE, None, 2, 4, 100, 4, 2, FAKE, FAKE, FAKE)
    need = rtopk.rtopk_workspace_bytes(2, 4, 100, 4, 1)
    assert need > 0
    assert rtopk.rtopk_beam_step_ws(*args, None, need, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_beam_step_ws(*args, FAKE + 8, need, None) == rtopk.RTOPK_EINVAL  # not 256-aligned
    assert rtopk.rtopk_beam_step_ws(*args, FAKE, need - 1, None) == rtopk.RTOPK_ENOMEM
    assert "smaller" in rtopk.rtopk_last_error()
    dbg = (None,) * 5
    assert rtopk.rtopk_debug_step(*args, FAKE, need - 256, *dbg, None) == rtopk.RTOPK_ENOMEM
    assert rtopk.rtopk_workspace_bytes(0, 4, 100, 4, 1) == 0


def test_last_error_is_thread_local(lib):
    import threading
    _step(B=0)
    seen = {}

    def other():
        seen["msg"] = rtopk.rtopk_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "sizes" in rtopk.rtopk_last_error()


@pytest.mark.parametrize("shape", [
    (2, 2, 8, 2, 0), (8, 4, 32000, 4, 0), (32, 4, 40000, 4, 1), (128, 4, 40000, 4, 1),
    (64, 8, 250000, 8, 2), (1, 1, 1, 1, 0), (3, 5, 1001, 3, 1), (2, 16, 5000, 64, 2), (7, 3, 37, 5, 0),
])
def test_plan_covers_rows(lib, shape):
    B, beam, V, k, dt = shape
    for mis in (0, 1, 3):
        esz = 4 if dt == 0 else 2
        base = None if mis == 0 else FAKE + mis * esz
        st, p = rtopk.rtopk_plan(base, B, beam, V, k, dt)
        assert st == 0, rtopk.rtopk_last_error()
        epv = 16 // esz
        assert p.elems_per_vec == epv and p.threads == 64
        assert p.align_elems == (mis % epv)
        span = (p.align_elems + V + epv - 1) // epv if (p.align_elems or V % epv) else V // epv
        # every vector a row touches lies in one of its pieces
        assert p.chunks * p.vecs_per_chunk >= span + (1 if (p.align_elems or V % epv) else 0) - 1
        assert p.vecs_per_chunk == p.threads * p.vecs_per_thread
        assert p.grid == -(-B * beam * p.chunks // p.pieces_per_group)
        assert p.ngroups >= k and p.ngroups & (p.ngroups - 1) == 0 and p.ngroups < 2 * k
        assert p.chunk_limit >= k
        assert p.queue_cap == beam * p.chunks * k
        assert p.sort_keys & (p.sort_keys - 1) == 0 and p.sort_keys <= 512
        assert p.sort_keys >= min(512, p.queue_cap + beam)
        assert p.row_local == (1 if p.pieces_per_group % p.chunks == 0 else 0)
        if p.row_local:  # the pieces' LDS regions, then every candidate of the workgroup
            assert p.lds_bytes >= p.pieces_per_group * 8 * (64 + k + 1) + 8 * p.pieces_per_group * (k + 1)
        else:
            assert p.lds_bytes >= 8 * p.sort_keys + 13 * beam + 13 * beam * p.chunks
        need = rtopk.rtopk_workspace_bytes(B, beam, V, k, dt)
        assert need >= 8 * B * p.queue_cap + 16 * B * beam * p.chunks


def test_overrides(lib):
    try:
        assert rtopk.rtopk_set_override(5, 0) == rtopk.RTOPK_EINVAL
        assert rtopk.rtopk_set_override(0, 129) == rtopk.RTOPK_EINVAL
        assert rtopk.rtopk_set_override(0, -1) == rtopk.RTOPK_EINVAL
        assert rtopk.rtopk_set_override(4, 1) == 0
        st, p = rtopk.rtopk_plan(None, 4, 4, 40000, 4, 1)
        assert st == 0 and p.vecs_per_thread == 4 and p.chunk_limit == 4  # raised to k
        assert p.chunks == math.ceil(5000 / (64 * 4))
    finally:
        rtopk.rtopk_set_override(0, 0)
    st, p = rtopk.rtopk_plan(None, 4, 4, 40000, 4, 1)
    assert p.chunk_limit == 128


def test_row_local_switch(lib):
    st, p = rtopk.rtopk_plan(None, 128, 4, 40000, 4, 1)
    assert st == 0 and p.chunks == 8 and p.pieces_per_group == 16 and p.row_local == 1
    try:
        assert rtopk.rtopk_set_row_local(0) == 0
        st, q = rtopk.rtopk_plan(None, 128, 4, 40000, 4, 1)
        assert st == 0 and q.row_local == 0 and q.chunks == p.chunks and q.grid == p.grid
    finally:
        rtopk.rtopk_set_row_local(1)
    st, p = rtopk.rtopk_plan(None, 3, 5, 1001, 3, 1)  # one piece per row: row-local too
    assert st == 0 and p.row_local == (1 if p.pieces_per_group % p.chunks == 0 else 0)


def test_split_switch(lib):
    assert rtopk.rtopk_set_split(0) == 0
    assert rtopk.rtopk_set_split(1) == 0


def test_release_without_workspaces_is_harmless(lib):
    rtopk.rtopk_release()


def test_read_probe_validation(lib):
    # misaligned source, ragged size and NULL pointers are rejected before any launch
    assert rtopk.rtopk_read_probe(0x1008, 64, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe(0x1000, 72, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe(None, 64, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe(0x1000, 64, 0, None, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe_shape(0x1000, 64, 3, 256, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe_shape(0x1000, 64, 4, 96, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe_shape(0x1000, 64, 4, 2048, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert rtopk.rtopk_read_probe_shape(0x1008, 64, 4, 256, 0, 0x2000, None) == rtopk.RTOPK_EINVAL
    assert "read probe" in rtopk.rtopk_last_error()


@pytest.mark.parametrize("shards,nshards_override,Vs,eos,msg", [
    (None, None, 8, 0, "shards is NULL"),
    ([0x1000] * 9, None, 8, 0, "nshards"),
    ([0x1000, 0], None, 8, 0, "shard 1 is NULL"),
    ([0x1000, 0x2008], None, 8, 0, "not 16-byte aligned"),
    ([0x1000, 0x2000], None, 5, 0, "multiple of 16"),
    ([0x1000, 0x2000], None, 8, 16, "eos_id"),
    ([0x1000, 0x2000], None, 0, 0, "V_shard"),
])
def test_sharded_validation_rejects_before_launch(lib, shards, nshards_override, Vs, eos, msg):
    st = rtopk.rtopk_beam_step_sharded(shards, rtopk.RTOPK_F16, 0x3000, None, 2, 2, Vs, 2, eos,
                                       0x4000, 0x5000, 0x6000, None)
    assert st == rtopk.RTOPK_EINVAL, rtopk.rtopk_last_error()
    assert msg in rtopk.rtopk_last_error()


def test_planner_workgroup_rules(lib):
    # grids that run in rounds (more pieces than 16 per CU on 256 CUs) use 8-wave workgroups
    st, p = rtopk.rtopk_plan(None, 64, 8, 250000, 8, 2)
    assert st == 0 and 64 * 8 * p.chunks > 4096 and p.pieces_per_group == 8  # B*beam*chunks pieces
    # with k >= 16, a row-local workgroup holds one batch element instead of several
    st, p = rtopk.rtopk_plan(None, 512, 1, 40000, 40, 1)
    assert st == 0 and p.row_local == 1 and p.pieces_per_group == p.chunks == 8
    st, p = rtopk.rtopk_plan(None, 512, 1, 40000, 8, 1)  # small k keeps 16-piece workgroups
    assert st == 0 and p.row_local == 1 and p.pieces_per_group == 16
    st, p = rtopk.rtopk_plan(None, 128, 4, 40000, 4, 1)  # the 4 x 40000 fp16 shape: 2 rows per workgroup
    assert st == 0 and p.row_local == 1 and p.chunks == 8 and p.pieces_per_group == 16 and p.grid == 256


def test_binding_rejects_host_logits():
    import torch
    from beam_search_top_amd import rtopk
    x = torch.zeros((2, 3, 16), dtype=torch.float16)
    a = torch.zeros((2, 3), dtype=torch.float32)
    with pytest.raises(ValueError):
        rtopk.beam_step(x, a, None, k=2)


def test_planner_small_row_local_grids(lib):
    # fewer row-local workgroups than CUs: whole batch elements per workgroup
    # when they fit, else one row per workgroup
    st, p = rtopk.rtopk_plan(None, 2, 2, 8, 2, 0)  # 2 x 2 x 8: one piece per row, batch element = 2 pieces
    assert st == 0 and p.row_local == 1 and p.pieces_per_group == 2 and p.grid == 2
    st, p = rtopk.rtopk_plan(None, 32, 4, 40000, 4, 1)  # 8 pieces per row, 32 per batch element
    assert st == 0 and p.row_local == 1 and p.pieces_per_group == 8 and p.grid == 128
    st, p = rtopk.rtopk_plan(None, 3, 4, 40000, 4, 1)
    assert st == 0 and p.row_local == 1 and p.pieces_per_group == 8
    st, p = rtopk.rtopk_plan(None, 128, 4, 40000, 4, 1)  # a full grid keeps 16-piece workgroups
    assert st == 0 and p.pieces_per_group == 16 and p.grid == 256
