"""Thin ctypes binding of librtopk.so (declared in include/rtopk.h).

The ``rtopk_*`` functions take integer device addresses and sizes, exactly like
the C ABI, and return its status codes. ``beam_step`` marshals torch tensors
(torch is used only for device memory and the current stream) and raises on a
non-OK status. Every step of the selection runs in the HIP kernels; there is no
fallback: without a built librtopk.so the import of this module's functions
fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librtopk.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "rtopk.h")

RTOPK_F32, RTOPK_F16, RTOPK_BF16 = 0, 1, 2
RTOPK_OK, RTOPK_EINVAL, RTOPK_ENOTSUP, RTOPK_ENOMEM, RTOPK_EHIP, RTOPK_ETIMEOUT = 0, -1, -2, -3, -4, -5
RTOPK_MAX_K, RTOPK_MAX_BEAM = 64, 512
RTOPK_WS_FIXED_BYTES = 1310976
RTOPK_NOALLOC_SCRATCH_BYTES = 8388608
RTOPK_DEFAULT_SPIN_LIMIT = 1 << 22
STATUS_NAMES = {0: "RTOPK_OK", -1: "RTOPK_EINVAL", -2: "RTOPK_ENOTSUP", -3: "RTOPK_ENOMEM", -4: "RTOPK_EHIP",
                -5: "RTOPK_ETIMEOUT"}


class RtopkError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class rtopk_plan_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "chunks", "threads", "vecs_per_thread", "vecs_per_chunk", "elems_per_vec", "ngroups",
        "chunk_limit", "queue_cap", "align_elems", "grid", "sort_keys", "lds_bytes", "pieces_per_group",
        "row_local")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load():
    """Load librtopk.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m beam_search_top_amd._build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    step_args = [vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.rtopk_beam_step.argtypes = step_args + [vp]
    L.rtopk_beam_step.restype = i32
    L.rtopk_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.rtopk_workspace_bytes.restype = sz
    L.rtopk_beam_step_ws.argtypes = step_args + [vp, sz, vp]
    L.rtopk_beam_step_ws.restype = i32
    L.rtopk_beam_step_noalloc.argtypes = step_args + [vp]
    L.rtopk_beam_step_noalloc.restype = i32
    L.rtopk_debug_step.argtypes = step_args + [vp, sz, vp, vp, vp, vp, vp, vp]
    L.rtopk_debug_step.restype = i32
    L.rtopk_plan.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(rtopk_plan_t)]
    L.rtopk_plan.restype = i32
    L.rtopk_set_override.argtypes = [i32, i32]
    L.rtopk_set_override.restype = i32
    L.rtopk_set_row_local.argtypes = [i32]
    L.rtopk_set_row_local.restype = i32
    L.rtopk_set_split.argtypes = [i32]
    L.rtopk_set_split.restype = i32
    L.rtopk_set_waves.argtypes = [i32]
    L.rtopk_set_waves.restype = i32
    L.rtopk_set_spin_limit.argtypes = [ctypes.c_uint]
    L.rtopk_set_spin_limit.restype = i32
    L.rtopk_check.argtypes = [vp, vp]
    L.rtopk_check.restype = i32
    L.rtopk_beam_step_sharded.argtypes = [ctypes.POINTER(vp), i32, i32, vp, vp, i32, i32, i32, i32, i32,
                                          vp, vp, vp, vp]
    L.rtopk_beam_step_sharded.restype = i32
    L.rtopk_sample_step.argtypes = [vp, i32, i32, i32, i32, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64,
                                    vp, vp, vp]
    L.rtopk_sample_step.restype = i32
    L.rtopk_lmhead_step.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.rtopk_lmhead_step.restype = i32
    L.rtopk_beam_reorder.argtypes = [vp, vp, ctypes.c_longlong, i32, i32, ctypes.c_longlong, vp, i32, vp]
    L.rtopk_beam_reorder.restype = i32
    L.rtopk_read_probe.argtypes = [vp, sz, ctypes.c_uint32, vp, vp]
    L.rtopk_read_probe.restype = i32
    L.rtopk_read_probe_shape.argtypes = [vp, sz, i32, i32, ctypes.c_uint32, vp, vp]
    L.rtopk_read_probe_shape.restype = i32
    L.rtopk_last_error.argtypes = []
    L.rtopk_last_error.restype = ctypes.c_char_p
    L.rtopk_release.argtypes = []
    L.rtopk_release.restype = None
    _lib = L
    return L


def declared_functions(header=HEADER):
    """Names of the functions include/rtopk.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtopk_[a-z0-9_]+)\s*\(", text)))


# ------------------------------------------------------------------ C-ABI mirror
def rtopk_beam_step(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                    out_beam_ids, out_token_ids, out_scores, stream):
    return load().rtopk_beam_step(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                                  out_beam_ids, out_token_ids, out_scores, stream)


def rtopk_workspace_bytes(B, beam, V, k, dtype):
    return load().rtopk_workspace_bytes(B, beam, V, k, dtype)


def rtopk_beam_step_ws(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                       out_beam_ids, out_token_ids, out_scores, workspace, ws_bytes, stream):
    return load().rtopk_beam_step_ws(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                                     out_beam_ids, out_token_ids, out_scores, workspace, ws_bytes, stream)


def rtopk_beam_step_noalloc(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                            out_beam_ids, out_token_ids, out_scores, stream):
    return load().rtopk_beam_step_noalloc(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                                          out_beam_ids, out_token_ids, out_scores, stream)


def rtopk_debug_step(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                     out_beam_ids, out_token_ids, out_scores, workspace, ws_bytes,
                     dbg_T, dbg_hits, dbg_lse, dbg_count, dbg_queue, stream):
    return load().rtopk_debug_step(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id,
                                   out_beam_ids, out_token_ids, out_scores, workspace, ws_bytes,
                                   dbg_T, dbg_hits, dbg_lse, dbg_count, dbg_queue, stream)


def rtopk_plan(logits, B, beam, V, k, dtype):
    """Returns (status, rtopk_plan_t)."""
    p = rtopk_plan_t()
    st = load().rtopk_plan(logits, B, beam, V, k, dtype, ctypes.byref(p))
    return st, p


def rtopk_set_override(vecs_per_thread, chunk_limit):
    return load().rtopk_set_override(vecs_per_thread, chunk_limit)


def rtopk_set_row_local(enable):
    return load().rtopk_set_row_local(enable)


def rtopk_set_split(enable):
    return load().rtopk_set_split(enable)


def rtopk_set_waves(waves):
    return load().rtopk_set_waves(waves)


def rtopk_set_spin_limit(polls):
    return load().rtopk_set_spin_limit(polls)


def rtopk_check(workspace, stream):
    return load().rtopk_check(workspace, stream)


def rtopk_beam_step_sharded(shards, dtype, alive_scores, finished_mask, B, beam, V_shard, k, eos_id,
                            out_beam_ids, out_token_ids, out_scores, stream):
    """`shards` is a Python sequence of device addresses (marshalled into the host array)."""
    arr = (ctypes.c_void_p * len(shards))(*shards) if shards is not None else None
    return load().rtopk_beam_step_sharded(arr, len(shards) if shards is not None else 0, dtype, alive_scores,
                                          finished_mask, B, beam, V_shard, k, eos_id, out_beam_ids,
                                          out_token_ids, out_scores, stream)


def beam_step_sharded(shards, alive, finished=None, k=None, eos_id=2):
    """One selection step over vocabulary shards (torch device tensors
    [B, beam, V_shard] of one dtype, shard g holding vocabulary indices
    g*V_shard ...), on the current stream. Returns (beam_ids, token_ids, scores)."""
    import torch
    s0 = shards[0]
    if any(t.shape != s0.shape or t.dtype != s0.dtype or not t.is_contiguous() for t in shards):
        raise ValueError("shards must be contiguous tensors of one shape and dtype")
    if not s0.is_cuda:
        raise ValueError("shards must be device tensors")
    for g, t in enumerate(shards):
        _on_device(t, s0.device, f"shard {g}")
    if k is None:
        k = s0.shape[1]
    B, beam, Vs = s0.shape
    _, _, _, finished, outs = _prepare(s0, alive, finished, k)
    stream = torch.cuda.current_stream(s0.device).cuda_stream
    _check(rtopk_beam_step_sharded([_ptr(t) for t in shards], dtype_code(s0), _ptr(alive), _ptr(finished),
                                   B, beam, Vs, k, eos_id, _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), stream))
    return outs


def rtopk_sample_step(logits, dtype, R, V, k, temperature, seed, step, out_token, out_logprob, stream):
    return load().rtopk_sample_step(logits, dtype, R, V, k, temperature, seed, step, out_token, out_logprob,
                                    stream)


def sample_step(logits, k, temperature=1.0, seed=0, step=0):
    """Top-k sampling of every row of logits [R, V] (torch device tensor) on
    the current stream. Returns (tokens [R] int32, logprobs [R] float32)."""
    import torch
    if logits.dim() != 2 or not logits.is_contiguous() or not logits.is_cuda:
        raise ValueError("logits must be a contiguous [R, V] device tensor")
    R, V = logits.shape
    tok = torch.empty(R, dtype=torch.int32, device=logits.device)
    lp = torch.empty(R, dtype=torch.float32, device=logits.device)
    stream = torch.cuda.current_stream(logits.device).cuda_stream
    _check(rtopk_sample_step(_ptr(logits), dtype_code(logits), R, V, k, float(temperature), int(seed), int(step),
                             _ptr(tok), _ptr(lp), stream))
    return tok, lp


def rtopk_lmhead_step(hidden, weight, alive_scores, finished_mask, B, beam, H, V, k, eos_id,
                      out_beam_ids, out_token_ids, out_scores, stream):
    return load().rtopk_lmhead_step(hidden, weight, alive_scores, finished_mask, B, beam, H, V, k, eos_id,
                                    out_beam_ids, out_token_ids, out_scores, stream)


def lmhead_step(hidden, weight, alive, finished=None, k=None, eos_id=2):
    """The step fused into the LM head, on torch device tensors (current
    stream): hidden [B*beam, H] and weight [V, H] bfloat16, alive [B, beam]
    float32, finished [B, beam] bool/uint8 or None. Returns (beam_ids,
    token_ids, scores), each [B, k]."""
    import torch
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden must be [B*beam, H] and weight [V, H]")
    if not (hidden.is_contiguous() and weight.is_contiguous()) or not hidden.is_cuda:
        raise ValueError("hidden and weight must be contiguous device tensors")
    dev = hidden.device
    _on_device(weight, dev, "weight")
    _on_device(alive, dev, "alive")
    if alive.dim() != 2 or alive.dtype != torch.float32 or not alive.is_contiguous():
        raise ValueError("alive must be a contiguous float32 [B, beam] tensor")
    B, beam = alive.shape
    if hidden.shape[0] != B * beam:
        raise ValueError("hidden must have B*beam rows")
    if finished is not None:
        _on_device(finished, dev, "finished")
        if finished.shape != (B, beam) or finished.dtype not in (torch.uint8, torch.bool):
            raise ValueError("finished must be a [B, beam] uint8/bool tensor")
        finished = finished.contiguous()
        if finished.dtype == torch.bool:
            finished = finished.view(torch.uint8)
    if k is None:
        k = beam
    V, H = weight.shape
    outs = (torch.empty((B, k), dtype=torch.int32, device=dev), torch.empty((B, k), dtype=torch.int32, device=dev),
            torch.empty((B, k), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(rtopk_lmhead_step(_ptr(hidden), _ptr(weight), _ptr(alive), _ptr(finished), B, beam, H, V, k, eos_id,
                             _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), stream))
    return outs


def rtopk_beam_reorder(src, dst, nslabs, B, beam, row_bytes, beam_ids, ld, stream):
    return load().rtopk_beam_reorder(src, dst, nslabs, B, beam, row_bytes, beam_ids, ld, stream)


def rtopk_read_probe(src, nbytes, marker, out, stream):
    return load().rtopk_read_probe(src, nbytes, marker, out, stream)


def rtopk_read_probe_shape(src, nbytes, vecs_per_lane, threads, marker, out, stream):
    return load().rtopk_read_probe_shape(src, nbytes, vecs_per_lane, threads, marker, out, stream)


def rtopk_last_error():
    return load().rtopk_last_error().decode()


def rtopk_release():
    load().rtopk_release()


# ------------------------------------------------------------------ torch marshalling
def _check(status):
    if status != RTOPK_OK:
        raise RtopkError(status, rtopk_last_error())


def dtype_code(t):
    import torch
    codes = {torch.float32: RTOPK_F32, torch.float16: RTOPK_F16, torch.bfloat16: RTOPK_BF16}
    if t.dtype not in codes:
        raise TypeError(f"logits dtype {t.dtype} is not float32/float16/bfloat16")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _on_device(t, dev, name):
    """Every tensor handed to the library must live on the logits' GPU: a host
    pointer in a kernel argument is a GPU memory fault, not an error code."""
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be a device tensor on {dev} (got {t.device})")


def _prepare(logits, alive, finished, k):
    import torch
    if logits.dim() != 3:
        raise ValueError("logits must be [B, beam, V]")
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    B, beam, V = logits.shape
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    dev = logits.device
    _on_device(alive, dev, "alive")
    if alive.shape != (B, beam) or alive.dtype != torch.float32 or not alive.is_contiguous():
        raise ValueError("alive must be a contiguous float32 [B, beam] tensor")
    if finished is not None:
        _on_device(finished, dev, "finished")
        if finished.shape != (B, beam) or finished.dtype not in (torch.uint8, torch.bool):
            raise ValueError("finished must be a [B, beam] uint8/bool tensor")
        finished = finished.contiguous()
        if finished.dtype == torch.bool:
            finished = finished.view(torch.uint8)
    outs = (torch.empty((B, k), dtype=torch.int32, device=dev),
            torch.empty((B, k), dtype=torch.int32, device=dev),
            torch.empty((B, k), dtype=torch.float32, device=dev))
    return B, beam, V, finished, outs


def _check_out(out, dev, B, k):
    """Caller-supplied outputs: (beam_ids int32, token_ids int32, scores float32), each [B, k]."""
    import torch
    if len(out) != 3:
        raise ValueError("out must hold three tensors (beam_ids, token_ids, scores)")
    for t, dt, name in zip(out, (torch.int32, torch.int32, torch.float32), ("beam_ids", "token_ids", "scores")):
        _on_device(t, dev, f"out {name}")
        if t.shape != (B, k) or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"out {name} must be a contiguous {dt} [{B}, {k}] tensor")
    return tuple(out)


def _check_workspace(ws, dev, need):
    import torch
    _on_device(ws, dev, "workspace")
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")


def beam_step(logits, alive, finished=None, k=None, eos_id=2, workspace=None, out=None):
    """One selection step on torch device tensors, on the current stream.

    logits [B, beam, V] float32/float16/bfloat16, alive [B, beam] float32,
    finished [B, beam] bool/uint8 or None. Returns (beam_ids, token_ids,
    scores), each [B, k]. ``workspace`` (a zero-filled uint8 device tensor of
    rtopk_workspace_bytes(...) bytes) selects rtopk_beam_step_ws; ``out`` may
    supply the three output tensors.
    """
    import torch
    if k is None:
        k = logits.shape[1]
    B, beam, V, finished, outs = _prepare(logits, alive, finished, k)
    if out is not None:
        outs = _check_out(out, logits.device, B, k)
    stream = torch.cuda.current_stream(logits.device).cuda_stream
    args = (_ptr(logits), dtype_code(logits), _ptr(alive), _ptr(finished), B, beam, V, k, eos_id,
            _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]))
    if workspace is not None:
        _check_workspace(workspace, logits.device, rtopk_workspace_bytes(B, beam, V, k, dtype_code(logits)))
    if workspace is None:
        _check(rtopk_beam_step(*args, stream))
    else:
        _check(rtopk_beam_step_ws(*args, _ptr(workspace), workspace.numel() * workspace.element_size(), stream))
    return outs


def beam_reorder(src, dst, beam_ids):
    """Cache refresh on torch device tensors, on the current stream.

    src, dst: contiguous [nslabs, B*beam, ...] tensors of one dtype (e.g. the
    keys and values of every layer stacked along dim 0); beam_ids: [B, ld]
    int32 with ld >= beam (rtopk_beam_step's beam ids with k = beam). New beam
    j of batch element b takes the row of old beam beam_ids[b, j]; an id
    outside [0, beam) leaves that row of dst as it was. Returns dst.
    """
    import torch
    if src.shape != dst.shape or src.dtype != dst.dtype or src.device != dst.device:
        raise ValueError("src and dst must have the same shape, dtype and device")
    if not src.is_cuda:
        raise ValueError("src and dst must be device tensors")
    _on_device(beam_ids, src.device, "beam_ids")
    if not (src.is_contiguous() and dst.is_contiguous() and beam_ids.is_contiguous()):
        raise ValueError("src, dst and beam_ids must be contiguous")
    if beam_ids.dtype != torch.int32 or beam_ids.dim() != 2 or src.dim() < 2:
        raise ValueError("beam_ids must be a [B, ld] int32 tensor and src at least 2-D")
    B, ld = beam_ids.shape
    if src.shape[1] % B != 0:
        raise ValueError("src.shape[1] must be B * beam")
    beam = src.shape[1] // B
    row_bytes = (src[0, 0].numel() if src.dim() > 2 else 1) * src.element_size()
    stream = torch.cuda.current_stream(src.device).cuda_stream
    _check(rtopk_beam_reorder(_ptr(src), _ptr(dst), src.shape[0], B, beam, row_bytes, _ptr(beam_ids), ld, stream))
    return dst


def debug_step(logits, alive, finished=None, k=None, eos_id=2):
    """beam_step plus the kernel's intermediate values (for tests).

    Returns a dict with the outputs and the plan, the per-piece thresholds
    T [B*beam*chunks], hit counts, merged lse [B*beam], per-batch queue
    counts and the raw queue [B, queue_cap] (uint64 entries).
    """
    import torch
    if k is None:
        k = logits.shape[1]
    B, beam, V, finished, outs = _prepare(logits, alive, finished, k)
    code = dtype_code(logits)
    st, plan = rtopk_plan(_ptr(logits), B, beam, V, k, code)
    _check(st)
    dev = logits.device
    nbytes = rtopk_workspace_bytes(B, beam, V, k, code)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    npieces = B * beam * plan.chunks
    dT = torch.full((npieces,), float("nan"), dtype=torch.float32, device=dev)
    dh = torch.zeros(npieces, dtype=torch.int32, device=dev)
    dl = torch.zeros(B * beam, dtype=torch.float32, device=dev)
    dc = torch.zeros(B, dtype=torch.int32, device=dev)
    dq = torch.zeros((B, plan.queue_cap), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(rtopk_debug_step(_ptr(logits), code, _ptr(alive), _ptr(finished), B, beam, V, k, eos_id,
                            _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(ws), nbytes,
                            _ptr(dT), _ptr(dh), _ptr(dl), _ptr(dc), _ptr(dq), stream))
    return dict(beam_ids=outs[0], token_ids=outs[1], scores=outs[2], plan=plan.as_dict(), T=dT, hits=dh,
                lse=dl, count=dc, queue=dq, workspace=ws)
