"""The step captured in a HIP graph (as the benchmark times it) and replayed:
every replay, with new logits copied into the captured input between replays
and eager work and synchronisations in between, gives the eager result."""
import numpy as np
import pytest
import torch

from beam_search_top_amd import rtopk, synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["b128", "c32k", "mixed250k"])
def test_graph_replays_match_eager(name):
    rtopk.load()
    L = rtopk.load()
    s = synth.make_step(name)
    x, a, f = to_device(s)
    nws = rtopk.rtopk_workspace_bytes(s.B, s.beam, s.V, s.k, s.dtype)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda:0")
    outs = [torch.empty((s.B, s.k), dtype=torch.int32, device="cuda:0"),
            torch.empty((s.B, s.k), dtype=torch.int32, device="cuda:0"),
            torch.empty((s.B, s.k), dtype=torch.float32, device="cuda:0")]
    xin = x.clone()

    def launch(stream):
        rc = L.rtopk_beam_step_ws(xin.data_ptr(), s.dtype, a.data_ptr(), f.data_ptr(), s.B, s.beam, s.V, s.k,
                                  s.eos_id, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                  ws.data_ptr(), nws, stream)
        assert rc == 0, rtopk.rtopk_last_error()

    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cs):
        launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    print(f"[graph] {name}", flush=True)
    for rep in range(4):
        xin.copy_(torch.roll(x, shifts=1237 * rep, dims=2))  # new logits in the captured buffer
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        launch(torch.cuda.current_stream().cuda_stream)  # eager, same inputs
        torch.cuda.synchronize()
        for g, e in zip(got, outs):
            assert torch.equal(g, e), (name, rep)
        assert (got[0] >= -1).all() and (got[0] < s.beam).all()
