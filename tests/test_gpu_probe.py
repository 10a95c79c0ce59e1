"""The ceiling probes (coli_probe_read, coli_probe_mfma) run through the C ABI,
leave their sink untouched and report plausible rates; they bound, rather
than take part in, the matmul path."""
import pytest
import torch

import bit_gemv_coli_amd as coli
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _timed(fn):
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    a.record(st)
    fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3


def test_probe_read_and_mfma():
    need_gpu()
    sink = torch.full((1,), 7.0, device="cuda")
    buf = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    t = _timed(lambda: coli.check(coli.coli_probe_read(buf, sink), "coli_probe_read"))
    gbs = buf.numel() / t / 1e9
    assert 500 < gbs < 20000, gbs
    wg, it = 1024, 200
    t = _timed(lambda: coli.check(coli.coli_probe_mfma(wg, it, sink), "coli_probe_mfma"))
    tf = wg * it * coli.PROBE_MFMA_FLOPS_PER_WG_ITER / t / 1e12
    assert 100 < tf < 3000, tf
    assert sink.item() == 7.0


def test_probe_declines_bad_arguments():
    need_gpu()
    sink = torch.zeros(1, device="cuda")
    buf = torch.ones(100, dtype=torch.uint8, device="cuda")  # not a multiple of 16 bytes
    assert coli.coli_probe_read(buf, sink) == coli.COLI_DECLINED
    assert coli.coli_probe_mfma(0, 10, sink) == coli.COLI_DECLINED
