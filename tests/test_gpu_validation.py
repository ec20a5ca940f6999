"""The Python binding rejects tensors on the wrong device (or of the wrong
type or size) with ValueError before anything is launched: a host pointer in
a kernel argument would be a GPU memory fault, not an error code."""
import numpy as np
import pytest
import torch

from beam_search_top_amd import rtopk, synth
from gpu_util import DEV, to_device
from libutil import ensure_built

pytestmark = pytest.mark.gpu


def _inputs():
    ensure_built()
    s = synth.make_custom(2, 3, 3, 1000, synth.F16, seed=1, sigma=2.0, n_finished=1)
    return s, to_device(s)


def _outs(B, k, device=DEV):
    return (torch.empty((B, k), dtype=torch.int32, device=device),
            torch.empty((B, k), dtype=torch.int32, device=device),
            torch.empty((B, k), dtype=torch.float32, device=device))


def test_host_or_mistyped_tensors_raise_before_launch():
    s, (x, a, f) = _inputs()
    cases = [
        dict(alive=a.cpu()),
        dict(finished=f.cpu()),
        dict(out=_outs(2, 3, device="cpu")),
        dict(out=(_outs(2, 3)[0], _outs(2, 3)[1], _outs(2, 3)[0])),  # scores as int32
        dict(out=_outs(2, 4)),                                       # wrong k
        dict(workspace=torch.zeros(rtopk.rtopk_workspace_bytes(2, 3, 1000, 3, 1), dtype=torch.uint8)),
        dict(workspace=torch.zeros(256, dtype=torch.uint8, device=DEV)),  # too small
        dict(workspace=torch.zeros(rtopk.rtopk_workspace_bytes(2, 3, 1000, 3, 1), dtype=torch.float32,
                                   device=DEV)),
    ]
    sentinel = _outs(2, 3)
    for t in sentinel:
        t.fill_(7)
    for kw in cases:
        args = dict(alive=a, finished=f)
        args.update(kw)
        with pytest.raises(ValueError):
            rtopk.beam_step(x, args["alive"], args["finished"], k=3, eos_id=2,
                            workspace=args.get("workspace"), out=args.get("out"))
    torch.cuda.synchronize()
    for t in sentinel:
        assert (t == 7).all()


def test_sharded_and_reorder_reject_host_tensors():
    s, (x, a, f) = _inputs()
    shards = [x[:, :, :500].contiguous(), x[:, :, 500:].contiguous()]
    with pytest.raises(ValueError):
        rtopk.beam_step_sharded([shards[0], shards[1].cpu()], a, f, k=3)
    with pytest.raises(ValueError):
        rtopk.beam_step_sharded(shards, a.cpu(), f, k=3)
    src = torch.zeros((2, 6, 64), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    ids = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        rtopk.beam_reorder(src, dst, ids.cpu())
    with pytest.raises(ValueError):
        rtopk.beam_reorder(src.cpu(), dst.cpu(), ids)
    with pytest.raises(ValueError):
        rtopk.sample_step(x[:, 0, :].contiguous().cpu(), k=3)
