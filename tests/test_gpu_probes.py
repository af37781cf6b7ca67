"""The measurement probes run, keep their results live and report clocks
that make sense (short runs; the figures themselves are the benchmark's)."""
import numpy as np
import pytest

from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


def test_probes_run_and_record_clocks(T):
    from trellis_quantized_linear_had_amd import _measure as _lib

    H.announce("probes: lds gather, mfma, streams (short)")
    L = _lib.mlib()
    sh = T.cuda.current_stream().cuda_stream
    sink = T.zeros(_lib.PROBE_SINK_BYTES, dtype=T.uint8, device="cuda")
    clocks = T.zeros(4 * _lib.PROBE_WORKGROUPS, dtype=T.int64, device="cuda")
    for fn in (L.exl3m_probe_lds_gather, L.exl3m_probe_mfma):
        clocks.zero_()
        _lib.check(fn(200, sink.data_ptr(), clocks.data_ptr(), sh))
        T.cuda.synchronize()
        c = clocks.cpu().numpy().view(np.uint64).reshape(-1, 4).astype(np.float64)
        assert np.all(c[:, 1] > c[:, 0]) and np.all(c[:, 3] > c[:, 2])
        ghz = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9
        assert np.all((ghz > 0.3) & (ghz < 3.0)), ghz[:4]
    n = 1 << 24
    buf = T.empty(n, dtype=T.uint8, device="cuda")
    _lib.check(L.exl3m_probe_stream(1, 0, buf.data_ptr(), n, sink.data_ptr(), sh))
    T.cuda.synchronize()
    words = buf.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.all(words[:, 1] == 0x3C003C00) and np.all(words[:, 3] == 0xFFFFFFFF)
    sink.zero_()
    _lib.check(L.exl3m_probe_stream(0, buf.data_ptr(), 0, n, sink.data_ptr(), sh))
    T.cuda.synchronize()
    assert sink.view(T.int32).abs().sum().item() > 0
    sink.zero_()
    # random bytes (the fill pattern's chunk indices cancel in the xor)
    g = T.Generator(device="cuda")
    g.manual_seed(7)
    rows = T.randint(0, 256, (10240 * 128 * 2,), dtype=T.uint8, device="cuda", generator=g)
    _lib.check(L.exl3m_probe_stream(2, rows.data_ptr(), 0, rows.numel(), sink.data_ptr(), sh))
    T.cuda.synchronize()
    assert sink.view(T.int32)[:128].abs().sum().item() > 0  # the two active waves of the one workgroup
    with pytest.raises(ValueError):
        _lib.check(L.exl3m_probe_stream(0, buf.data_ptr(), 0, 24, sink.data_ptr(), sh))
