"""Graph capture of the C-ABI calls: a call captured into a HIP graph (through
torch.cuda.graph on its capture stream) and replayed must give the eager
result bit for bit on every replay, also after the inputs are overwritten in
place and with unrelated eager work between replays. The calls allocate
nothing, synchronize nothing and take every buffer from the caller, which is
what capture needs (vLLM PR #314, "Problem": lazily allocated state breaks
capture; the decode-shaped calls are the ones a serving loop captures)."""
import numpy as np
import pytest

import workloads as WL
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


def _linear_call(torch, lib, layer, x, y, scratch, M, pm):
    return lambda: lib.exl3_linear(layer.c, x.data_ptr(), M, y.data_ptr(), scratch.data_ptr(), scratch.numel(), pm,
                                   torch.cuda.current_stream().cuda_stream)


def _replays_match_eager(torch, call, inputs, outputs, fresh_inputs, other_work):
    """Eager run, capture, then three replays with new input contents; every
    replay is compared with an eager run on the same inputs."""
    from trellis_quantized_linear_had_amd import _lib

    _lib.check(call())  # eager (also caches the device check before capture)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _lib.check(call())  # warm-up on a side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(g):
        status.append(call())
    assert status == [0]
    for rep in range(3):
        for dst, src in zip(inputs, fresh_inputs(rep)):
            dst.copy_(src)
        torch.cuda.synchronize()
        _lib.check(call())
        torch.cuda.synchronize()
        eager = [o.clone() for o in outputs]
        for o in outputs:
            o.fill_(0x5A5A if o.dtype == torch.int16 else -7)  # stale results must not survive
        torch.cuda.synchronize()
        g.replay()
        other_work()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), "replay %d differs from the eager result" % rep


@pytest.mark.parametrize("M,pm", [(1, 128), (2, 128), (4, 128), (8, 128), (16, 128), (64, 128), (256, 128),
                                  (1100, 128)])
def test_linear_graph_replay_bit_identical(T, M, pm):
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib

    H.announce("graph capture exl3_linear K1024 N2048 M=%d" % M)
    K, N = 1024, 2048
    cb = WL.codebook()
    layer = X.Layer.from_numpy(WL.layer(29, K, N), cb)
    other = X.Layer.from_numpy(WL.layer(29, K, N, 1), cb)
    x = _lib.to_device_u16(WL.activations(29, M, K))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    scratch = torch.empty(X.linear_scratch_bytes(K, N, M, pm), dtype=torch.uint8, device="cuda")
    # unrelated eager work between replays: another layer into other buffers
    y2 = torch.empty_like(y)
    s2 = torch.empty_like(scratch)
    call = _linear_call(torch, _lib.lib(), layer, x, y, scratch, M, pm)
    call2 = _linear_call(torch, _lib.lib(), other, x, y2, s2, M, pm)
    fresh = lambda rep: [_lib.to_device_u16(WL.activations(29, M, K, 100 + rep))]
    _replays_match_eager(torch, call, [x], [y], fresh, lambda: _lib.check(call2()))


def test_logits_graph_replay_bit_identical(T):
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib

    H.announce("graph capture logits_pad_mask_argmax M=16 K512 w_rows 1000 n_valid 777")
    M, K, w_rows, n_valid = 16, 512, 1000, 777
    rng = np.random.default_rng(30)
    x = _lib.to_device_u16((0.05 * rng.standard_normal((M, K))).astype(np.float16).view(np.uint16))
    w = _lib.to_device_u16((0.02 * rng.standard_normal((w_rows, K))).astype(np.float16).view(np.uint16))
    n_pad = X.logits_padded_width(n_valid, w_rows)
    lg = torch.empty((M, n_pad), dtype=torch.int16, device="cuda")
    am = torch.empty(M, dtype=torch.int64, device="cuda")
    scratch = torch.empty(X.logits_scratch_bytes(M, K, n_valid, w_rows), dtype=torch.uint8, device="cuda")
    L = _lib.lib()

    def call():
        return L.logits_pad_mask_argmax(x.data_ptr(), M, K, w.data_ptr(), w_rows, n_valid, lg.data_ptr(), n_pad,
                                        am.data_ptr(), scratch.data_ptr(), scratch.numel(),
                                        torch.cuda.current_stream().cuda_stream)

    def fresh(rep):
        r = np.random.default_rng(31 + rep)
        return [_lib.to_device_u16((0.05 * r.standard_normal((M, K))).astype(np.float16).view(np.uint16))]

    _replays_match_eager(torch, call, [x], [lg, am], fresh, lambda: torch.cuda.synchronize())


@pytest.mark.parametrize("M,pm", [(1, 128), (16, 128), (256, 128)])
def test_head_graph_replay_bit_identical(T, M, pm):
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib

    H.announce("graph capture exl3_head_logits_argmax K512 N2048 n_valid 1500 M=%d" % M)
    K, N, n_valid = 512, 2048, 1500
    cb = WL.codebook()
    layer = X.Layer.from_numpy(WL.layer(32, K, N, 0, 6), cb)
    x = _lib.to_device_u16(WL.activations(32, M, K))
    n_pad = X.logits_padded_width(n_valid, N)
    lg = torch.empty((M, n_pad), dtype=torch.int16, device="cuda")
    am = torch.empty(M, dtype=torch.int64, device="cuda")
    scratch = torch.empty(X.head_scratch_bytes(K, N, M, n_valid, pm), dtype=torch.uint8, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.int16, device="cuda")
    s2 = torch.empty(X.linear_scratch_bytes(K, N, M, pm), dtype=torch.uint8, device="cuda")
    L = _lib.lib()

    def call():
        return L.exl3_head_logits_argmax(layer.c, x.data_ptr(), M, n_valid, lg.data_ptr(), n_pad, am.data_ptr(),
                                         scratch.data_ptr(), scratch.numel(), pm,
                                         torch.cuda.current_stream().cuda_stream)

    other = _linear_call(torch, L, layer, x, y2, s2, M, pm)
    fresh = lambda rep: [_lib.to_device_u16(WL.activations(32, M, K, 200 + rep))]
    _replays_match_eager(torch, call, [x], [lg, am], fresh, lambda: _lib.check(other()))
