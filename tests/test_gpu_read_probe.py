"""The plain-read ceiling probe (a measurement aid of bench.py) reads every byte
it is given: it finds a marker word wherever it is placed, and reports nothing
when the marker is absent."""
import pytest
import torch

from beam_search_top_amd import rtopk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 40_960_000, 41_000_016])
def test_read_probe_sees_every_word(nbytes):
    rtopk.load()
    n = nbytes // 4
    buf = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    marker = 0x13579BDF
    assert rtopk.rtopk_read_probe(buf.data_ptr(), nbytes, marker, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert out.item() == 0
    for pos in sorted({0, n // 3, n - 1}):
        buf[pos] = marker
        out.zero_()
        assert rtopk.rtopk_read_probe(buf.data_ptr(), nbytes, marker, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert out.item() == 1, pos
        buf[pos] = 0


@pytest.mark.parametrize("vecs,threads", [(1, 64), (4, 256), (10, 512), (16, 1024)])
@pytest.mark.parametrize("nbytes", [16, 1_000_016, 41_000_016])
def test_read_probe_shape_sees_every_word(vecs, threads, nbytes):
    rtopk.load()
    n = nbytes // 4
    buf = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    marker = 0x2468ACE1
    assert rtopk.rtopk_read_probe_shape(buf.data_ptr(), nbytes, vecs, threads, marker, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert out.item() == 0
    for pos in sorted({0, n // 2, n - 1}):
        buf[pos] = marker
        out.zero_()
        assert rtopk.rtopk_read_probe_shape(buf.data_ptr(), nbytes, vecs, threads, marker, out.data_ptr(),
                                            stream) == 0
        torch.cuda.synchronize()
        assert out.item() == 1, pos
        buf[pos] = 0
