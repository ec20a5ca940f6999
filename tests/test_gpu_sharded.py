"""The step over vocabulary shards (rtopk_beam_step_sharded): every shard its
own tensor, merged per beam and batch element inside one launch. It must give
the oracle's result on the concatenated vocabulary."""
import numpy as np
import pytest
import torch

from beam_search_top_amd import rtopk, synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def _check(s, got):
    from test_gpu_parity import check
    check(s, got)


def _split(x, G):
    Vs = x.shape[2] // G
    return [x[:, :, g * Vs:(g + 1) * Vs].contiguous() for g in range(G)]


@pytest.mark.parametrize("name,G", [("b128", 2), ("b128", 4), ("b128", 8), ("c32k", 4), ("tiny", 2),
                                    ("spiked40k", 5), ("mixed250k", 2), ("mixed250k", 5)])
def test_sharded_matches_oracle(name, G):
    s = synth.make_step(name)
    print(f"[sharded] {name} G={G}", flush=True)
    x, a, f = to_device(s)
    got = rtopk.beam_step_sharded(_split(x, G), a, f, k=s.k, eos_id=s.eos_id)
    torch.cuda.synchronize()
    _check(s, tuple(t.cpu().numpy() for t in got))
    # the unsharded step on the same logits picks the same pairs
    ref = rtopk.beam_step(x, a, f, k=s.k, eos_id=s.eos_id)
    torch.cuda.synchronize()
    assert np.array_equal(got[0].cpu().numpy(), ref[0].cpu().numpy())
    assert np.array_equal(got[1].cpu().numpy(), ref[1].cpu().numpy())


@pytest.mark.parametrize("G,Vs,k,dt", [(3, 8, 5, synth.F16), (7, 1024, 8, synth.BF16), (2, 4, 1, synth.F32),
                                       (8, 64000, 4, synth.F16)])
def test_sharded_custom_shapes(G, Vs, k, dt):
    s = synth.make_custom(3, 4, k, G * Vs, dt, seed=G * 100 + k, n_finished=2)
    print(f"[sharded] custom G={G} Vs={Vs} k={k} dtype={dt}", flush=True)
    x, a, f = to_device(s)
    got = rtopk.beam_step_sharded(_split(x, G), a, f, k=s.k, eos_id=s.eos_id)
    torch.cuda.synchronize()
    _check(s, tuple(t.cpu().numpy() for t in got))
