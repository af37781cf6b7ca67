"""The Python binding rejects what the C ABI cannot see (it receives bare
pointers): wrong shapes, dtypes, strides, devices and undersized buffers
raise ValueError naming the condition, before any library call. CPU only:
the checks run before the device check, and the device check (every tensor
on the layer's GPU) is the last to fire here."""
import numpy as np
import pytest
import torch

import workloads as WL
from trellis_quantized_linear_had_amd import _lib as B


@pytest.fixture(scope="module")
def layer():
    return B.Layer.from_numpy(WL.layer(WL.SEED_TINY, 256, 384), WL.codebook(), device="cpu")


def x16(M, K):
    return torch.zeros((M, K), dtype=torch.int16)


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_layer_tensors_are_checked():
    spec = WL.layer(WL.SEED_TINY, 256, 384)
    cb = WL.codebook()
    raises("codes holds", B.Layer, spec["codes"][:-1], cb, spec["scale"], K=256, N=384, device="cpu")
    raises("codebook holds", B.Layer, spec["codes"], cb[:65535], spec["scale"], K=256, N=384, device="cpu")
    raises("scale holds", B.Layer, spec["codes"], cb, spec["scale"][:383], K=256, N=384, device="cpu")
    raises("sign_k holds", B.Layer, spec["codes"], cb, spec["scale"], spec["sign_k"][:255], K=256, N=384,
           device="cpu")
    raises("multiples of 128", B.Layer, spec["codes"], cb, spec["scale"], K=200, N=384, device="cpu")
    raises("bits = 9", B.Layer, spec["codes"], cb, spec["scale"], K=256, N=384, bits=9, device="cpu")
    f32 = torch.zeros(384, dtype=torch.float32)
    raises("scale has dtype", B.Layer, spec["codes"], cb, f32, K=256, N=384, device="cpu")
    # 6 bits need 1.5x the 4-bit code words
    raises("codes holds", B.Layer, spec["codes"], cb, spec["scale"], K=256, N=384, bits=6, device="cpu")


def test_linear_rejects_bad_activations_and_buffers(layer):
    raises("2-D", B.linear, torch.zeros(256, dtype=torch.int16), layer)
    raises("columns; the layer takes K = 256", B.linear, x16(4, 128), layer)
    raises("dtype", B.linear, torch.zeros((4, 256), dtype=torch.float32), layer)
    raises("contiguous", B.linear, x16(256, 4).t(), layer)
    raises("out has shape", B.linear, x16(4, 256), layer, out=x16(4, 256))
    raises("scratch has dtype", B.linear, x16(4, 256), layer, scratch=torch.zeros(10, dtype=torch.float32))
    raises("must be on a GPU", B.linear, x16(4, 256), layer)


def test_head_rejects_bad_arguments(layer):
    raises("n_valid = 0", B.head_logits_argmax, x16(2, 256), layer, 0)
    raises("n_valid = 385", B.head_logits_argmax, x16(2, 256), layer, 385)
    raises("logits must be", B.head_logits_argmax, x16(2, 256), layer, 300, logits=x16(2, 128))
    raises("argmax has dtype", B.head_logits_argmax, x16(2, 256), layer, 300,
           argmax=torch.zeros(2, dtype=torch.int32))
    raises("argmax holds", B.head_logits_argmax, x16(2, 256), layer, 300, argmax=torch.zeros(1, dtype=torch.int64))
    raises("must be on a GPU", B.head_logits_argmax, x16(2, 256), layer, 300)


def test_logits_rejects_bad_arguments():
    w = x16(300, 256)
    raises("w must be a 2-D", B.logits_pad_mask_argmax, x16(2, 256), torch.zeros(10, dtype=torch.int16), 5)
    raises("columns; the layer takes K = 256", B.logits_pad_mask_argmax, x16(2, 128), w, 257)
    raises("logits has", B.logits_pad_mask_argmax, x16(2, 256), w, 257, logits=x16(2, 257))
    raises("argmax holds", B.logits_pad_mask_argmax, x16(2, 256), w, 257,
           argmax=torch.zeros(1, dtype=torch.int64))
    raises("must be on a GPU", B.logits_pad_mask_argmax, x16(2, 256), w, 257)


def test_had_and_reconstruct_reject_bad_arguments(layer):
    raises("x must be a 2-D", B.had_r_128, torch.zeros(128, dtype=torch.int16))
    raises("sign_pre holds", B.had_r_128, x16(2, 256), sign_pre=torch.zeros(128, dtype=torch.int16))
    raises("out has shape", B.had_r_128, x16(2, 256), out=x16(2, 128))
    raises("must be on a GPU", B.had_r_128, x16(2, 256))
    raises("unknown layout", B.reconstruct, layer, layout=5)
    raises("out has shape", B.reconstruct, layer, out=x16(256, 128))
    raises("must be on a GPU", B.reconstruct, layer, out=x16(256, 384))


def test_scratch_size_is_checked_before_the_call(layer):
    need = B.linear_scratch_bytes(256, 384, 4)
    assert need > 0
    small = torch.zeros(need - 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="must be on a GPU"):  # the device check comes first for x
        B.linear(x16(4, 256), layer, scratch=small)
    with pytest.raises(ValueError, match="this call needs"):
        B._scratch(small, need, torch.device("cpu"), None)
    assert np.isscalar(need)
