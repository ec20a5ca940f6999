"""Device-side helpers for the GPU tests: move a synth.Step to cuda:0 and run
the HIP path through the C ABI (via the ctypes binding)."""
import numpy as np
import torch

from beam_search_top_amd import rtopk, synth
from libutil import ensure_built

DEV = "cuda:0"


def logits_tensor(s, device=DEV):
    if s.dtype == synth.F32:
        t = torch.from_numpy(np.ascontiguousarray(s.logits))
    elif s.dtype == synth.F16:
        t = torch.from_numpy(np.ascontiguousarray(s.logits))
    else:
        t = torch.from_numpy(np.ascontiguousarray(s.logits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def to_device(s, device=DEV):
    return (logits_tensor(s, device), torch.from_numpy(s.alive).to(device),
            torch.from_numpy(s.finished).to(device))


def run(s, finished=True, **kw):
    ensure_built()
    x, a, f = to_device(s)
    out = rtopk.beam_step(x, a, f if finished else None, k=s.k, eos_id=s.eos_id, **kw)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def misaligned_copy(s, offset, device=DEV):
    """Logits placed `offset` elements past a 256-byte-aligned allocation."""
    x = logits_tensor(s, device)
    buf = torch.empty(x.numel() + offset + 64, dtype=x.dtype, device=device)
    view = buf[offset:offset + x.numel()].view(x.shape)
    view.copy_(x)
    return view
