"""Cache refresh on the GPU (rtopk_beam_reorder through the C ABI) against the
oracle's definition, byte for byte."""
import numpy as np
import pytest
import torch

import oracle
from beam_search_top_amd import rtopk

pytestmark = pytest.mark.gpu


def _case(nslabs, B, beam, row_bytes, seed, ld=None, offset=0, pad_frac=0.1):
    rng = np.random.default_rng(seed)
    ld = ld or beam
    total = nslabs * B * beam * row_bytes
    src_h = rng.integers(0, 256, size=total, dtype=np.uint8)
    dst_h = rng.integers(0, 256, size=total, dtype=np.uint8)
    ids = rng.integers(0, beam, size=(B, ld)).astype(np.int32)
    ids[rng.random((B, ld)) < pad_frac] = -1
    return src_h, dst_h, ids, offset


@pytest.mark.parametrize("nslabs,B,beam,row_bytes,offset", [
    (1, 1, 1, 16, 0), (2, 3, 4, 48, 0), (12, 8, 4, 65536, 0), (3, 5, 3, 16400, 0),
    (2, 2, 8, 1, 0), (2, 4, 3, 7, 0), (4, 3, 5, 16 * 1024 + 3, 0), (2, 3, 4, 64, 5), (6, 16, 4, 4096, 16),
])
def test_reorder_matches_oracle(nslabs, B, beam, row_bytes, offset):
    rtopk.load()
    src_h, dst_h, ids, off = _case(nslabs, B, beam, row_bytes, seed=nslabs * 1000 + row_bytes, offset=offset)
    n = src_h.size
    print(f"[reorder] nslabs={nslabs} B={B} beam={beam} row_bytes={row_bytes} offset={off}", flush=True)
    src = torch.zeros(n + 64, dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda:0")
    src[off:off + n] = torch.from_numpy(src_h).cuda()
    dst[off:off + n] = torch.from_numpy(dst_h).cuda()
    guard_before = dst[:off].clone(), dst[off + n:].clone()
    idt = torch.from_numpy(ids).cuda()
    st = rtopk.rtopk_beam_reorder(src.data_ptr() + off, dst.data_ptr() + off, nslabs, B, beam, row_bytes,
                                  idt.data_ptr(), ids.shape[1], torch.cuda.current_stream().cuda_stream)
    assert st == 0, rtopk.rtopk_last_error()
    torch.cuda.synchronize()
    want = oracle.beam_reorder(src_h, dst_h, ids, nslabs, B, beam).reshape(-1)
    got = dst[off:off + n].cpu().numpy()
    assert np.array_equal(got, want)
    assert torch.equal(dst[:off], guard_before[0]) and torch.equal(dst[off + n:], guard_before[1])


def test_reorder_ld_wider_than_beam_and_torch_wrapper():
    # beam ids of a selection with k > beam (ld = k): only the first beam columns are used
    rtopk.load()
    nslabs, B, beam, k = 4, 6, 3, 5
    x = torch.randn(nslabs, B * beam, 8, 32, dtype=torch.float16, device="cuda:0")
    y = torch.randn_like(x)
    ids = torch.randint(-1, beam, (B, k), dtype=torch.int32, device="cuda:0")
    before = y.clone()
    rtopk.beam_reorder(x, y, ids)
    torch.cuda.synchronize()
    want = oracle.beam_reorder(x.cpu().view(torch.uint8).numpy(), before.cpu().view(torch.uint8).numpy(),
                               ids.cpu().numpy(), nslabs, B, beam)
    assert np.array_equal(y.cpu().view(torch.uint8).numpy().reshape(want.shape), want)


def test_reorder_after_a_selection_step():
    # the full decode-step tail: select with k = beam, then refresh the cache by the selected beams
    from beam_search_top_amd import synth
    s = synth.make_custom(8, 4, 4, 4000, synth.F16, seed=90, n_finished=3)
    x = torch.from_numpy(s.logits).cuda()
    a = torch.from_numpy(s.alive).cuda()
    f = torch.from_numpy(s.finished).cuda()
    bi, ti, sc = rtopk.beam_step(x, a, f, k=s.k, eos_id=s.eos_id)
    cache = torch.randn(2 * 3, s.B * s.beam, 4, 16, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(cache)
    rtopk.beam_reorder(cache, out, bi)
    torch.cuda.synchronize()
    ref = oracle.step_of(s)
    assert np.array_equal(bi.cpu().numpy(), ref.beam_ids)
    want = oracle.beam_reorder(cache.cpu().view(torch.uint8).numpy(), out.cpu().view(torch.uint8).numpy(),
                               ref.beam_ids, 6, s.B, s.beam)
    assert np.array_equal(out.cpu().view(torch.uint8).numpy().reshape(want.shape), want)
