"""GPU parity of every entry point against the CPU oracle, through the C ABI,
at sizes the oracle finishes in seconds that still span several tiles and
ragged tails."""
import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


@pytest.fixture(scope="module")
def X(T):
    import trellis_quantized_linear_had_amd as X

    return X


@pytest.fixture(scope="module")
def cb():
    return WL.codebook()


def dev16(a):
    from trellis_quantized_linear_had_amd import _lib

    return _lib.to_device_u16(a)


def host16(t):
    from trellis_quantized_linear_had_amd import _lib

    return _lib.to_host_u16(t)


# ------------------------------------------------------------------ Hadamard

@pytest.mark.parametrize("rows,cols,pre,post", [
    (1, 128, False, False), (3, 512, True, False), (37, 5120, True, True), (5, 17408, False, True),
    (1000, 256, True, True),
])
def test_had_r_128_matches_oracle(T, X, rows, cols, pre, post):
    H.announce("had_r_128 rows=%d cols=%d pre=%d post=%d" % (rows, cols, pre, post))
    x = WL.activations(11, rows, cols)
    sp = WL.signs(11, 2, cols) if pre else None
    sq = WL.signs(11, 3, cols) if post else None
    ref = O.had128(x, sp, sq)
    got = host16(X.had_r_128(dev16(x), None if sp is None else dev16(sp), None if sq is None else dev16(sq)))
    d = H.ulp_diff(got, ref)
    assert d.max() <= 1, d.max()
    assert np.mean(d > 0) < 1e-3


def test_had_r_128_in_place_and_involution(T, X):
    H.announce("had_r_128 in place")
    x = WL.activations(12, 64, 1024)
    t = dev16(x)
    X.had_r_128(t, out=t)
    assert H.ulp_diff(host16(t), O.had128(x)).max() <= 1
    X.had_r_128(t, out=t)
    xv, back = H.val(x), H.val(host16(t))
    assert np.max(np.abs(back - xv)) <= 2.0 ** -9 * np.max(np.abs(xv))


# ------------------------------------------------------------ trellis decode

@pytest.mark.parametrize("K,N", [(128, 128), (256, 256), (5120, 384), (384, 1152)])
def test_decode_states_bit_exact(T, X, cb, K, N):
    H.announce("decode_states K=%d N=%d" % (K, N))
    L = WL.layer(21, K, N)
    lay = X.Layer.from_numpy(L, cb)
    got = host16(X.decode_states(lay))
    assert np.array_equal(got, O.trellis_states(L["codes"], K, N))


def test_decode_states_closed_form_tile(T, X, cb):
    H.announce("decode_states closed form")
    K = N = 128
    codes = np.full(K * N // 8, 0x76543210, np.uint32)
    L = {"codes": codes, "scale": np.full(N, 0x3C00, np.uint16), "K": K, "N": N}
    got = host16(X.decode_states(X.Layer.from_numpy(L, cb)))
    # nibble q of every tile is q mod 8, so state(i) = nibbles i..i+3 (mod 8)
    for k in (0, 1, 4, 5, 7):
        n = 3
        i = 16 * n + k
        expect = sum(((i + u) % 8) << (4 * u) for u in range(4))
        assert got[k, n] == expect


@pytest.mark.parametrize("K,N,n0,nc", [(256, 256, 0, 256), (256, 384, 128, 48), (5120, 512, 16, 480),
                                       (128, 33024, 32768, 256)])
def test_reconstruct_kn_bit_exact(T, X, cb, K, N, n0, nc):
    H.announce("reconstruct KN K=%d N=%d n0=%d nc=%d" % (K, N, n0, nc))
    L = WL.layer(22, K, N)
    lay = X.Layer.from_numpy(L, cb)
    got = host16(X.reconstruct(lay, n0, nc, X.LAYOUT_KN))
    assert np.array_equal(got, O.reconstruct(L["codes"], cb, L["scale"], K, N, n0, nc))


@pytest.mark.parametrize("K,N,n0,nc,pad", [(256, 256, 0, 256, 0), (384, 512, 128, 272, 24), (5120, 1024, 0, 1024, 0)])
def test_reconstruct_nk_bit_exact(T, X, cb, K, N, n0, nc, pad):
    H.announce("reconstruct NK K=%d N=%d n0=%d nc=%d pad=%d" % (K, N, n0, nc, pad))
    L = WL.layer(23, K, N)
    lay = X.Layer.from_numpy(L, cb)
    out = T.full((nc, K + pad), -1, dtype=T.int16, device="cuda")
    X.reconstruct(lay, n0, nc, X.LAYOUT_NK, out=out, ldw=K + pad)
    got = host16(out)
    ref = O.reconstruct(L["codes"], cb, L["scale"], K, N, n0, nc)
    assert np.array_equal(got[:, :K], ref.T)
    assert np.all(got[:, K:] == 0xFFFF)  # padding columns untouched


def test_reconstruct_identity_codebooks_recover_states(T, X):
    H.announce("reconstruct identity codebooks")
    K, N = 256, 384
    L = WL.layer(24, K, N)
    s = np.arange(65536)
    L["scale"] = np.full(N, 0x3C00, np.uint16)
    lo = H.val(host16(X.reconstruct(X.Layer.from_numpy(L, (s & 255).astype(np.float16).view(np.uint16)))))
    hi = H.val(host16(X.reconstruct(X.Layer.from_numpy(L, (s >> 8).astype(np.float16).view(np.uint16)))))
    states = (hi * 256 + lo).astype(np.int64)
    assert np.array_equal(states, O.trellis_states(L["codes"], K, N).astype(np.int64))


# ------------------------------------------------------------------- layer

def run_linear(X, L, cb, x, pm):
    lay = X.Layer.from_numpy(L, cb)
    return host16(X.linear(dev16(x), lay, prefill_min_m=pm))


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 47, 48, 64, 65, 127, 128, 129, 130, 191, 192, 300, 1024, 1025])
def test_linear_tiny_every_route(T, X, cb, M):
    """Each kernel sequence (forced) against the oracle, and the dispatch:
    the default threshold, 0 (fused side only) and 1 (prefill side only)
    each give the forced output of the sequence the rule names, bit for bit."""
    H.announce("linear tiny K256 N256 M=%d" % M)
    K = N = 256
    L = WL.layer(WL.SEED_TINY, K, N)
    lay = X.Layer.from_numpy(L, cb)
    x = WL.activations(WL.SEED_TINY, M, K)
    ref = O.exl3_linear(x, L, cb)
    out = {r: H.linear_forced(lay, x, r) for r in ("fused", "recon", "dq", "dq8")}
    for r, y in out.items():
        H.assert_rows_close(y, ref, what=r)
    H.assert_rows_close(out["fused"], out["recon"], what="fused vs recon")
    for pm in (128, 0, 1):
        assert np.array_equal(run_linear(X, L, cb, x, pm), out[H.route(4, M, pm)]), pm


def test_linear_deterministic(T, X, cb):
    H.announce("linear determinism")
    K, N = 1024, 2048
    L = WL.layer(25, K, N)
    for M, pm in ((16, 128), (256, 128)):
        x = WL.activations(25, M, K)
        a = run_linear(X, L, cb, x, pm)
        b = run_linear(X, L, cb, x, pm)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("K,N,M", [(5120, 17408, 2048), (2560, 3328, 200)])
def test_prefill_gemm_repeatable(T, X, cb, K, N, M):
    """Back-to-back prefill calls (full tiles plus stream-K pieces at the
    first shape, pieces straddling tiles at the second) give the same bits
    every time: the GEMM's operand loads and their waits leave no call
    reading a stage or fragment before it has landed."""
    H.announce("prefill repeatable K%d N%d M%d" % (K, N, M))
    import torch

    from trellis_quantized_linear_had_amd import _measure

    L = WL.layer(26, K, N)
    lay = X.Layer.from_numpy(L, cb)
    x = dev16(WL.activations(26, M, K))
    scr = torch.empty(_measure.linear_scratch_bytes(K, N, M, _measure.VARIANT_RECON_GEMM), dtype=torch.uint8,
                      device="cuda")
    outs = [torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(8)]
    for o in outs:  # reconstruct + GEMM forced (at M = 200 the dispatch picks the dequant-GEMM)
        H.linear_forced(lay, x, "recon", out=o, scratch=scr, sync=False)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_linear_two_slices(T, X, cb):
    H.announce("linear two 32768-column slices K128 N33024 M130")
    K, N, M = 128, 33024, 130
    L = WL.layer(26, K, N)
    x = WL.activations(26, M, K)
    rows = np.array([0, 1, 64, 128, 129], np.int64)
    ref = O.exl3_linear(x, L, cb, rows)
    got = H.linear_forced(X.Layer.from_numpy(L, cb), x, "recon")
    H.assert_rows_close(got[rows], ref)


@pytest.mark.parametrize("K,N,M", [
    (2560, 3328, 200),    # 13 tiles < 256 CUs: the tail as 26 256x128 halves, pieces of 5 k-steps over 40
                          # straddling halves; each tile's second half is ragged (rows 128..199 of 256)
    (2560, 3328, 100),    # the same split with every second half past the last row (q 128..255, M = 100):
                          # those pieces read clamped rows and their fixup stores nothing
    (1024, 4352, 4096),   # 272 tiles: one whole round + 16 tiles as 32 halves split along K
    (1024, 4608, 300),    # 36 tiles in two column blocks, the last ragged: grouped tail order (3-strip groups)
])
def test_linear_prefill_gemm_tail(T, X, cb, K, N, M):
    H.announce("linear prefill GEMM tail K%d N%d M%d" % (K, N, M))
    L = WL.layer(28, K, N)
    x = WL.activations(28, M, K)
    rows = np.unique(np.array([0, 1, 31, 32, 127, 128, 255, 256, 257, M // 2, M - 2, M - 1], np.int64) % M)
    ref = O.exl3_linear(x, L, cb, rows)
    lay = X.Layer.from_numpy(L, cb)
    got = H.linear_forced(lay, x, "recon")
    H.assert_rows_close(got[rows], ref)
    again = H.linear_forced(lay, x, "recon")
    assert np.array_equal(got, again)  # the piece order is fixed: bit-identical reruns


def test_empty_calls_are_noops(T, X, cb):
    """M = 0 (and a zero-row rotation) returns OK and leaves the outputs as
    they were."""
    import torch

    from trellis_quantized_linear_had_amd import _lib

    H.announce("empty calls")
    K, N = 256, 384
    lay = X.Layer.from_numpy(WL.layer(32, K, N), cb)
    x = dev16(WL.activations(32, 4, K))
    y = torch.full((4, N), 0x1234, dtype=torch.int16, device="cuda")
    scratch = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    L = _lib.lib()
    for pm in (0, 1, 128):
        assert L.exl3_linear(lay.c, x.data_ptr(), 0, y.data_ptr(), scratch.data_ptr(), scratch.numel(), pm, sh) == 0
    assert L.had_r_128(x.data_ptr(), y.data_ptr(), 0, K, None, None, sh) == 0
    w = dev16(np.zeros((300, K), np.uint16))
    am = torch.full((4,), -5, dtype=torch.int64, device="cuda")
    assert L.logits_pad_mask_argmax(x.data_ptr(), 0, K, w.data_ptr(), 300, 257, y.data_ptr(), N, am.data_ptr(),
                                    scratch.data_ptr(), scratch.numel(), sh) == 0
    torch.cuda.synchronize()
    assert bool((y == 0x1234).all()) and bool((am == -5).all())


def test_linear_zero_codes_rank_one(T, X, cb):
    """All-zero codes: every weight is fp16(cb[0] * scale[n]) (the oracle's
    rank-1 closed form is pinned on the CPU); both paths against the oracle."""
    H.announce("linear all-zero codes K512 N640")
    K, N = 512, 640
    L = WL.layer(33, K, N)
    L["codes"] = np.zeros_like(L["codes"])
    lay = X.Layer.from_numpy(L, cb)
    for M in (3, 130):
        x = WL.activations(33, M, K)
        ref = O.exl3_linear(x, L, cb)
        for r in ("fused", "recon", "dq", "dq8"):
            H.assert_rows_close(H.linear_forced(lay, x, r), ref, what="%s M=%d" % (r, M))


def test_linear_without_signs(T, X, cb):
    H.announce("linear without sign vectors")
    K, N, M = 256, 384, 20
    L = WL.layer(27, K, N)
    L["sign_k"] = None
    L["sign_n"] = None
    ones_k = np.full(K, 0x3C00, np.uint16)
    ones_n = np.full(N, 0x3C00, np.uint16)
    ref = O.exl3_linear(WL.activations(27, M, K), dict(L, sign_k=ones_k, sign_n=ones_n), cb)
    x = WL.activations(27, M, K)
    H.assert_rows_close(run_linear(X, L, cb, x, 0), ref)
    H.assert_rows_close(run_linear(X, L, cb, x, 1), ref)


# ------------------------------------------------------------------ logits

def run_logits(X, x, w, n_valid):
    lg, am = X.logits_pad_mask_argmax(dev16(x), dev16(w), n_valid)
    return host16(lg), am.cpu().numpy()


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M,K,w_rows,n_valid", [(3, 256, 300, 257), (16, 512, 1000, 777), (17, 128, 640, 640),
                                                (1, 5120, 4096, 3001), (2, 256, 130, 1)])
def test_logits_match_oracle(T, X, M, K, w_rows, n_valid):
    H.announce("logits M=%d K=%d w_rows=%d n_valid=%d" % (M, K, w_rows, n_valid))
    r = np.random.default_rng(M * 7 + K)
    x = f16(0.05 * r.standard_normal((M, K)))
    w = f16(0.02 * r.standard_normal((w_rows, K)))
    ref_lg, ref_am = O.logits(x, w, n_valid)
    lg, am = run_logits(X, x, w, n_valid)
    n_pad = O.padded_width(n_valid, w_rows)
    assert lg.shape == (M, n_pad)
    assert np.all(lg[:, n_valid:] == 0xFC00)
    H.assert_logits_close(lg[:, :n_valid], ref_lg[:, :n_valid], K)
    assert np.array_equal(am, ref_am)
    # the argmax is the first maximum of the logits the kernel returned
    assert np.array_equal(am, np.argmax(H.val(lg), axis=1))


def test_logits_planted_pad_row_nan_poison_and_ties(T, X):
    H.announce("logits planted row, NaN poison, ties")
    r = np.random.default_rng(5)
    M, K, w_rows, n_valid = 4, 256, 520, 300   # n_pad = 384
    x = f16(0.05 * r.standard_normal((M, K)))
    w = f16(0.02 * r.standard_normal((w_rows, K)))
    w[310] = f16(5 * H.val(x[0]))       # wins row 0 if the mask were missing
    w[384:] = 0x7E00                    # NaN beyond the padded width: never read
    w[350] = 0x7E00                     # NaN inside the pad region: masked
    _, am0 = O.logits(x, w, n_valid)    # the oracle never reads rows at or past n_valid
    lg, am = run_logits(X, x, w, n_valid)
    assert np.array_equal(am, am0)
    assert np.all(lg[:, n_valid:] == 0xFC00)
    # ties: duplicate every row's winner at a higher and a lower index
    w2 = w.copy()
    for i in range(M):
        b = int(am[i])
        w2[min(b + 1 + i, n_valid - 1)] = w2[b]
        w2[max(b - 1 - i, 0)] = w2[b]
    lg2, am2 = run_logits(X, x, w2, n_valid)
    v = H.val(lg2)
    for i in range(M):
        assert am2[i] == np.min(np.nonzero(v[i] == v[i].max())[0])


def test_logits_nan_rule(T, X):
    """NaN logits: the first NaN wins (NumPy's and torch's argmax), also over
    +inf; a row whose decodable logits are all NaN selects column 0, never a
    pad column. Same inputs as the oracle's pin."""
    from tests.test_oracle_logits import nan_logits_case

    H.announce("logits NaN rule")
    x, w = nan_logits_case()
    for wv in (w, np.concatenate([np.full((1, w.shape[1]), 0x7E00, np.uint16), w[1:]]),
               np.concatenate([np.full((300, w.shape[1]), 0x7E00, np.uint16), w[300:]])):
        lg, am = run_logits(X, x, wv, 300)
        _, ref_am = O.logits(x, wv, 300)
        assert np.array_equal(am, ref_am), (am, ref_am)
        assert np.array_equal(am, np.argmax(H.val(lg), axis=1))
        assert np.all(am < 300) and np.all(lg[:, 300:] == 0xFC00)


def test_logits_aligned_width_mask_is_noop(T, X):
    H.announce("logits aligned width")
    r = np.random.default_rng(6)
    x = f16(0.05 * r.standard_normal((2, 256)))
    w = f16(0.02 * r.standard_normal((512, 256)))
    lg, am = run_logits(X, x, w, 384)
    assert lg.shape == (2, 384)
    assert not np.any(lg == 0xFC00)
    ref_lg, ref_am = O.logits(x, w, 384)
    assert np.array_equal(am, ref_am)


@pytest.mark.parametrize("M,route", [(1, None), (16, None), (130, None), (130, "recon"), (64, "fused")])
def test_linear_largest_k(T, X, cb, M, route):
    """K = 65408, the largest K the library takes (an fp16 weight slice of
    K x 32768 columns stays within 32-bit byte offsets), on every route
    (the dispatch's at M = 1, 16 and 130, the others forced)."""
    H.announce("linear K65408 N256 M=%d route=%s" % (M, route))
    K, N = 65408, 256
    L = WL.layer(27, K, N)
    x = WL.activations(27, M, K)
    y = run_linear(X, L, cb, x, 128) if route is None else H.linear_forced(X.Layer.from_numpy(L, cb), x, route)
    rows = np.unique(np.array([0, M // 2, M - 1], np.int64))
    H.assert_rows_close(y[rows], O.exl3_linear(x, L, cb, rows))
