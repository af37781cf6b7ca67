"""The C-ABI library loads, exports every declared symbol, and its pure host
functions and argument validation behave as declared (no GPU needed: every
call here returns before any device work)."""
import ctypes
import os
import re

import pytest

from trellis_quantized_linear_had_amd import _lib as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "exl3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    decl = declared_functions()
    assert set(decl) == set(X.EXPORTS), decl
    L = X.lib()
    for name in decl:
        assert hasattr(L, name), name


def test_padded_width_rule():
    assert X.lib().logits_padded_width(248077, 248320) == 248192
    assert X.lib().logits_padded_width(256, 1000) == 256
    assert X.lib().logits_padded_width(257, 300) == 300
    assert X.lib().logits_padded_width(0, 10) == -1
    assert X.lib().logits_padded_width(11, 10) == -1


TAIL_MAX = (256 + 223) * 256 * 256 * 4


def test_scratch_sizes():
    L = X.lib()
    # Wide projection: fp16 rotated input (M x K) + one 32768-column fp16 slice of W.
    wide = L.exl3_linear_scratch_bytes(5120, 32768, 2048, 128)
    assert wide == 2048 * 5120 * 2 + 5120 * 32768 * 2
    assert 5120 * 32768 * 2 == 335544320  # the 336 MB bound of the pages' 32768-column slicing
    # N above one slice still holds a single slice (plus the fp32 k-piece tiles
    # of the GEMM's stream-K tail: one 256x256 fp32 tile per (piece, tile)
    # pair, at most 256 pieces + 223 tile boundaries inside pieces)
    two = L.exl3_linear_scratch_bytes(128, 33024, 128, 128)
    assert 128 * 128 * 2 + 32768 * 128 * 2 <= two <= 128 * 128 * 2 + 32768 * 128 * 2 + TAIL_MAX
    # decode path is used below the threshold and when the threshold is 0
    d = L.exl3_linear_scratch_bytes(5120, 17408, 16, 128)
    assert d == L.exl3_linear_scratch_bytes(5120, 17408, 16, 0)
    assert d > 16 * 5120 * 2
    # M at the threshold takes the prefill path: rotated input + the whole 17408-column slice
    pre = L.exl3_linear_scratch_bytes(5120, 17408, 16, 16)
    assert 16 * 5120 * 2 + 17408 * 5120 * 2 <= pre <= 16 * 5120 * 2 + 17408 * 5120 * 2 + TAIL_MAX
    assert L.exl3_linear_scratch_bytes(100, 128, 1, 128) == 0
    assert L.exl3_linear_scratch_bytes(128, 128, 0, 128) == 0
    assert L.logits_scratch_bytes(16, 5120, 248077, 248320) >= 16 * 5120 * 2  # includes the fragment-ordered x
    assert L.logits_scratch_bytes(16, 5120, 0, 10) == 0
    assert L.logits_scratch_bytes(16, -128, 248077, 248320) == 0


def _layer(K=256, N=256, bits=4, codes=0x1000, cb=0x2000, scale=0x3000):
    return X.Exl3Layer(codes, cb, scale, None, None, K, N, bits)


def _linear(layer, x=0x4000, M=1, y=0x5000, scratch=0x6000, nbytes=1 << 30, pm=128):
    return X.lib().exl3_linear(ctypes.byref(layer), x, M, y, scratch, nbytes, pm, None)


@pytest.mark.parametrize("layer,status", [
    (_layer(K=100), X.EXL3_ESHAPE),
    (_layer(N=130), X.EXL3_ESHAPE),
    (_layer(bits=0), X.EXL3_ESHAPE),
    (_layer(bits=9), X.EXL3_ESHAPE),
    (_layer(K=65408, N=65792, bits=8), X.EXL3_ESHAPE),  # 8-bit codes past 4 GiB (4 bits would fit)
    (_layer(codes=0), X.EXL3_EINVAL),
    (_layer(cb=0), X.EXL3_EINVAL),
    (_layer(codes=0x1004), X.EXL3_EINVAL),
    (_layer(K=65536, N=128), X.EXL3_ESHAPE),          # K past the 32-bit slice addressing
    (_layer(K=65408, N=131584), X.EXL3_ESHAPE),       # packed codes past 4 GiB
])
def test_linear_rejects_bad_layers(layer, status):
    assert _linear(layer) == status
    assert X.lib().exl3_strerror(status)


def test_every_width_from_1_to_8_passes_validation():
    # validation passes, so the call gets as far as the scratch check
    for bits in range(1, 9):
        assert _linear(_layer(bits=bits), nbytes=0) == X.EXL3_ESCRATCH, bits
    assert _linear(_layer(K=65408, N=65792, bits=4), nbytes=0) == X.EXL3_ESCRATCH
    states = X.lib().exl3_decode_states
    assert states(ctypes.byref(_layer(bits=9)), 0x7000, None) == X.EXL3_ESHAPE
    assert states(ctypes.byref(_layer(bits=0)), 0x7000, None) == X.EXL3_ESHAPE


def test_linear_rejects_bad_calls():
    good = _layer()
    assert _linear(good, M=-1) == X.EXL3_EINVAL
    assert _linear(good, M=0) == X.EXL3_OK            # no-op
    assert _linear(good, x=0) == X.EXL3_EINVAL
    assert _linear(good, scratch=0) == X.EXL3_EINVAL
    assert _linear(good, scratch=0x6010) == X.EXL3_EINVAL   # scratch must be 256-byte aligned
    need = X.lib().exl3_linear_scratch_bytes(256, 256, 1, 128)
    assert _linear(good, nbytes=need - 1) == X.EXL3_ESCRATCH
    assert b"needs" in X.lib().exl3_strerror(X.EXL3_ESCRATCH)
    assert _linear(good, pm=-1) == X.EXL3_EINVAL
    # the prefill path addresses the rotated input with 32-bit offsets: M * K * 2 < 4 GiB
    big = _layer(K=65408, N=128)
    assert _linear(big, M=32833, pm=128) == X.EXL3_ESHAPE    # 32833 * 65408 * 2 > 2^32
    assert b"4 GiB" in X.lib().exl3_strerror(X.EXL3_ESHAPE)


def test_reconstruct_and_had_validation():
    L = X.lib()
    lay = _layer()
    assert L.exl3_reconstruct(ctypes.byref(lay), 8, 16, 0x7000, 16, 0, None) == X.EXL3_ESHAPE   # misaligned slice
    assert L.exl3_reconstruct(ctypes.byref(lay), 0, 272, 0x7000, 272, 0, None) == X.EXL3_ESHAPE  # beyond N
    assert L.exl3_reconstruct(ctypes.byref(lay), 0, 16, 0x7000, 8, 0, None) == X.EXL3_ESHAPE    # ldw < n_count
    assert L.exl3_reconstruct(ctypes.byref(lay), 0, 16, 0x7000, 128, 1, None) == X.EXL3_ESHAPE  # NK: ldw < K
    assert L.exl3_reconstruct(ctypes.byref(lay), 0, 16, 0x7000, 16, 5, None) == X.EXL3_EINVAL   # layout
    assert L.exl3_reconstruct(ctypes.byref(lay), 0, 0, 0x7000, 16, 0, None) == X.EXL3_OK        # empty slice
    assert L.had_r_128(0x1000, 0x2000, 4, 100, None, None, None) == X.EXL3_ESHAPE
    assert L.had_r_128(0x1000, 0x2000, -1, 128, None, None, None) == X.EXL3_EINVAL
    assert L.had_r_128(0, 0x2000, 4, 128, None, None, None) == X.EXL3_EINVAL
    assert L.had_r_128(0x1000, 0x2000, 0, 128, None, None, None) == X.EXL3_OK


def test_logits_validation():
    L = X.lib()

    def call(M=1, K=256, w_rows=300, n_valid=257, ld=300, nbytes=1 << 20, x=0x1000):
        return L.logits_pad_mask_argmax(x, M, K, 0x2000, w_rows, n_valid, 0x3000, ld, 0x4000, 0x5000, nbytes, None)

    assert call(n_valid=0) == X.EXL3_EWIDTH
    assert call(n_valid=301) == X.EXL3_EWIDTH
    assert call(ld=299) == X.EXL3_EWIDTH
    assert call(K=200) == X.EXL3_ESHAPE
    assert call(K=(1 << 23) + 128) == X.EXL3_ESHAPE  # a wave's 128 rows past a 32-bit buffer range
    assert call(M=-1) == X.EXL3_EINVAL
    assert call(x=0) == X.EXL3_EINVAL
    assert call(nbytes=0) == X.EXL3_ESCRATCH
    assert call(M=0) == X.EXL3_OK


def test_head_validation_and_scratch():
    L = X.lib()
    lay = _layer(K=256, N=1024)

    def call(M=1, n_valid=777, ld=896, nbytes=1 << 30, x=0x4000, logits=0x5000, argmax=0x8000, pm=128):
        return L.exl3_head_logits_argmax(ctypes.byref(lay), x, M, n_valid, logits, ld, argmax, 0x6000, nbytes, pm,
                                         None)

    assert call(n_valid=0) == X.EXL3_EWIDTH
    assert call(n_valid=1025) == X.EXL3_EWIDTH
    assert call(ld=888) == X.EXL3_EWIDTH        # below the padded width 896
    assert call(ld=900) == X.EXL3_EWIDTH        # not a multiple of 8
    assert call(M=-1) == X.EXL3_EINVAL
    assert call(x=0) == X.EXL3_EINVAL
    assert call(logits=0x5008) == X.EXL3_EINVAL  # 16-byte alignment
    assert call(argmax=0) == X.EXL3_EINVAL
    assert call(argmax=0x8004) == X.EXL3_EINVAL
    assert call(nbytes=0) == X.EXL3_ESCRATCH
    assert call(M=0) == X.EXL3_OK
    assert _linear(_layer(bits=9)) == X.EXL3_ESHAPE
    assert L.exl3_head_logits_argmax(ctypes.byref(_layer(N=130)), 0x4000, 1, 100, 0x5000, 256, 0x8000, 0x6000,
                                     1 << 30, 128, None) == X.EXL3_ESHAPE
    # scratch: the layer's first n_pad columns (decode partials or one prefill
    # slice), then one (fp32 max, int32 index) pair per row and 4096-column piece
    def extra(M, n_pad):
        pairs = M * -(-n_pad // 4096)
        return 2 * (-(-pairs * 4 // 256) * 256)

    def lin(n, M):
        return -(-L.exl3_linear_scratch_bytes(256, n, M, 128) // 256) * 256

    assert L.exl3_head_scratch_bytes(256, 1024, 16, 1024, 128) == lin(1024, 16) + extra(16, 1024)
    assert L.exl3_head_scratch_bytes(256, 1024, 16, 777, 128) == lin(896, 16) + extra(16, 896)
    assert L.exl3_head_scratch_bytes(256, 1024, 256, 100, 128) == lin(128, 256) + extra(256, 128)
    head = L.exl3_head_scratch_bytes(5120, 248320, 16, 248077, 128)
    base = L.exl3_linear_scratch_bytes(5120, 248192, 16, 128)
    assert base < head <= base + 256 + extra(16, 248192)
    assert L.exl3_head_scratch_bytes(256, 1024, 16, 0, 128) == 0
    assert L.exl3_head_scratch_bytes(256, 1024, 16, 1025, 128) == 0
    assert L.exl3_head_scratch_bytes(256, 1024, 0, 10, 128) == 0


def test_noalloc_refuses_oversize_before_any_device_work():
    """The size check of the allocation-free entry point comes before the
    device is touched: a prefill call far beyond its 48 MiB array is refused
    here, with no GPU."""
    L = X.lib()
    layer = X.Exl3Layer(0x1000, 0x1000, 0x1000, None, None, 5120, 17408, 4)
    st = L.exl3_linear_noalloc(ctypes.byref(layer), 0x1000, 2048, 0x2000, 128, None)
    assert st == X.EXL3_ESCRATCH
    assert "exl3_linear_noalloc holds 50331648" in L.exl3_strerror(st).decode()
    assert L.exl3_linear_noalloc(ctypes.byref(layer), None, 16, 0x2000, 128, None) == X.EXL3_EINVAL
    assert L.exl3_linear_noalloc(ctypes.byref(layer), 0x1000, 0, 0x2000, 128, None) == X.EXL3_OK
    assert X.NOALLOC_SCRATCH_BYTES == 48 * 1024 * 1024


def measure_declared_functions():
    src = open(os.path.join(ROOT, "trellis_quantized_linear_had_amd", "measure", "measure.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_product_library_holds_no_measurement_code():
    """The product library exports the C ABI of exl3.h and no timing hook or
    probe; those live in the separate measurement library."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", X.LIB_PATH], capture_output=True, text=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    c_names = {n for n in names if not n.startswith("_")}
    assert c_names == set(X.EXPORTS), sorted(c_names ^ set(X.EXPORTS))
    assert not any("probe" in n or "timer" in n for n in names)


def test_measure_library_exports_and_validation_without_gpu():
    from trellis_quantized_linear_had_amd import _measure as MS

    decl = measure_declared_functions()
    assert set(decl) == set(MS.EXPORTS), decl
    L = MS.mlib()
    for name in decl:
        assert hasattr(L, name), name
    assert L.exl3m_probe_lds_gather(-1, 0x1000, 0x2000, None) == X.EXL3_EINVAL
    assert L.exl3m_probe_mfma(10, 0, 0x2000, None) == X.EXL3_EINVAL
    assert L.exl3m_probe_stream(0, 0x1000, 0, 24, 0x2000, None) == X.EXL3_EINVAL   # not a multiple of 16
    assert L.exl3m_probe_stream(1, 0x1000, 0, 32, 0x2000, None) == X.EXL3_EINVAL   # write needs dst
    assert L.exl3m_probe_stream(0, 0x1000, 0, 0, 0x2000, None) == X.EXL3_OK        # nothing to stream
    assert L.exl3m_probe_stream(3, 0x1000, 0x1000, 32, 0x2000, None) == X.EXL3_EINVAL  # unknown mode
    assert L.exl3m_probe_stream(2, 0, 0x1000, 32, 0x2000, None) == X.EXL3_EINVAL   # row read needs src
    assert "misaligned" in L.exl3m_strerror(X.EXL3_EINVAL).decode()
    used = ctypes.c_int(-1)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    # an unknown mark kind, and event arrays missing: refused before the library call
    assert L.exl3m_linear_marked(None, None, 1, None, None, 0, 128, None, 7, 0, None, None,
                                 ctypes.byref(used), 0) == X.EXL3_EINVAL
    assert L.exl3m_linear_marked(None, None, 1, None, None, 0, 128, None, 0, 4, None, None,
                                 ctypes.byref(used), 0) == X.EXL3_EINVAL
    assert L.exl3m_linear_marked(None, None, 1, None, None, 0, 128, None, 0, 0, vpp(), vpp(),
                                 ctypes.byref(used), 9) == X.EXL3_EINVAL   # unknown variant
    # valid marks, then the library's own validation (NULL layer) speaks
    assert L.exl3m_linear_marked(None, None, 1, None, None, 0, 128, None, 0, 0, vpp(), vpp(),
                                 ctypes.byref(used), 0) == X.EXL3_EINVAL
    assert used.value == 0
    assert "layer is NULL" in L.exl3m_strerror(X.EXL3_EINVAL).decode()


def test_missing_library_fails_loudly():
    """Without libexl3.so the binding raises at first use: there is no CPU or
    PyTorch fallback behind the entry points."""
    import subprocess
    import sys

    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from trellis_quantized_linear_had_amd import _lib\n"
        "_lib.LIB_PATH = '/nonexistent/libexl3.so'\n"
        "import trellis_quantized_linear_had_amd as T\n"
        "try:\n"
        "    T.logits_padded_width(248077, 248320)\n"
        "except ImportError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout


@pytest.mark.parametrize("K,N,M", [
    (17408, 5120, 2048),  # 160 tiles, pieces of 170 k-steps straddling tiles of 272
    (5120, 17408, 2048),  # 32 tail tiles as 64 halves, 4 pieces of 20 k-steps per half
    (2560, 3328, 200),    # 13 tiles, pieces of 3 k-steps over 40
    (1024, 4608, 300),    # 36 tiles, pieces of 3 k-steps over 16
    (5120, 5120, 128),    # 20 tiles as 40 halves, 247 pieces of 13 k-steps over 80
    (1024, 4352, 4096),   # one whole round + 16 tiles split along K
    (5120, 17408, 4096),  # 1024 whole tiles + 64 split
    (256, 256, 128),      # one tile in 4 pieces of one k-step
])
def test_prefill_scratch_counts_every_piece_tile_pair(K, N, M):
    """The GEMM tail's partial region holds one fp32 accumulator tile per
    (piece, tail item) pair; the pairs are counted here by walking each
    piece's k-step run, independently of the library's closed-form slot
    count. Tail items are the 256x256 tail tiles, or their 256x128 halves when
    a piece over whole tiles would be at most an eighth of a tile's k-steps."""
    import math

    tiles = math.ceil(N / 256) * math.ceil(M / 256)
    rem = tiles % 256
    nk = K // 64
    pairs, split = 0, 1
    if 0 < rem <= 224 and nk >= 2:
        if 2 * rem <= 256 and 8 * math.ceil(rem * nk / 256) <= nk:
            split = 2
        total = rem * split * nk
        units = math.ceil(total / 256)
        for v in range(math.ceil(total / units)):
            lo, hi = v * units, min((v + 1) * units, total)
            pairs += len({u // nk for u in range(lo, hi)})
    a256 = lambda b: (b + 255) // 256 * 256
    base = a256(math.ceil(M / 32) * 32 * K * 2) + a256(N * K * 2)
    assert X.lib().exl3_linear_scratch_bytes(K, N, M, 1) == base + pairs * 256 * (256 // split) * 4
