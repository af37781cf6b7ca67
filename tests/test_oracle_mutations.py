"""The oracle's pins are sensitive to plausible mistakes: each mistake below,
planted in a temporary copy of the oracle source (never in the oracle
itself), is built with the oracle's own compiler flags, and the oracle pin
suite, run in a child process against that build, must fail. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_fp16.py", "tests/test_oracle_hadamard.py", "tests/test_oracle_trellis.py",
        "tests/test_oracle_trellis_bits.py", "tests/test_oracle_linear.py", "tests/test_oracle_logits.py",
        "tests/test_oracle_head.py"]

# (name, exact text in oracle.c, replacement): each replaced text occurs once.
MUTATIONS = [
    ("rounding_half_away", "double q = rint(ldexp(a, 10 - e));", "double q = floor(ldexp(a, 10 - e) + 0.5);"),
    ("subnormal_quantum", "double q = rint(ldexp(a, 24));", "double q = rint(ldexp(a, 23));"),
    ("hadamard_negated", "& 1) ? -1 : 1; }", "& 1) ? 1 : -1; }"),
    ("hadamard_or_index", "__builtin_popcount((unsigned)(i & j))", "__builtin_popcount((unsigned)(i | j))"),
    ("hadamard_norm_dropped", "acc *= norm;", "acc *= 1.0;"),
    ("window_off_by_one_bit", "(bits * i + t) % tile_len", "(bits * i + t + 1) % tile_len"),
    ("window_msb_first", "tile_bit(tile, (bits * i + t) % tile_len) << t;",
     "tile_bit(tile, (bits * i + t) % tile_len) << (15 - t);"),
    ("step_always_4_bits", "tile_bit(tile, (bits * i + t) % tile_len)", "tile_bit(tile, (4 * i + t) % tile_len)"),
    ("tile_length_fixed", "const int tile_len = 256 * bits;", "const int tile_len = 1024;"),
    ("steps_n_fastest", "(n % 16) * 16 + (k % 16)", "(k % 16) * 16 + (n % 16)"),
    ("neighbour_tile", "codes + (kt * (N / 16) + nt) * 8 * bits", "codes + ((kt * (N / 16) + nt) ^ 1) * 8 * bits"),
    ("tile_stride_fixed", "codes + (kt * (N / 16) + nt) * 8 * bits", "codes + (kt * (N / 16) + nt) * 32"),
    ("linear_bits_ignored", "oracle_reconstruct(codes, cb, scale, K, N, bits, 0, N, w);",
     "oracle_reconstruct(codes, cb, scale, K, N, 4, 0, N, w);"),
    ("scale_dropped", "* h2d(scale[n]); /* exact product */", "; /* exact product */"),
    ("scale_slice_column", "h2d(cb[weight_state(codes, N, (int)bits, k, n)]) * h2d(scale[n])",
     "h2d(cb[weight_state(codes, N, (int)bits, k, n)]) * h2d(scale[j])"),
    ("input_signs_ignored", "had_row(xin, sk, NULL, K, xh);", "had_row(xin, NULL, NULL, K, xh);"),
    ("output_signs_ignored", "had_row(yh, NULL, sn, N, yo);", "had_row(yh, NULL, NULL, N, yo);"),
    ("gemm_transposed_operand", "acc[n] += a * tab[wk[n]];", "acc[n] += a * tab[w[(n * N + k) % (K * N)]];"),
    ("xr_not_rounded", "xh[k] = tab[d2h(xh[k])];", "xh[k] = xh[k];"),
    ("yr_not_rounded", "yh[n] = tab[d2h(acc[n])];", "yh[n] = acc[n];"),
    ("pad_not_masked", "row[n] = 0xFC00; /* -inf */", "row[n] = 0x0000; /* -inf */"),
    ("argmax_last_maximum", "if (isnan(v) || v > bv) {", "if (isnan(v) || v >= bv) {"),
    ("argmax_nan_never_selected", "if (isnan(v) || v > bv) {", "if (v > bv) {"),
    ("argmax_last_nan_wins", "n < n_pad && !isnan(bv); ++n", "n < n_pad; ++n"),
    ("width_multiple_of_64", "(n_valid + 127) / 128 * 128", "(n_valid + 63) / 64 * 64"),
    ("head_row_stride", "memcpy(logits + i * n_pad, y + i * N,", "memcpy(logits + i * n_pad, y + i * n_pad,"),
    ("head_tail_columns", "y + i * N, (size_t)n_pad", "y + i * N + (N - n_pad), (size_t)n_pad"),
    ("head_mask_skipped", "argmax[i] = mask_and_select(logits + i * n_pad, n_valid, n_pad, tab);\n  }\n  free(y);",
     "argmax[i] = mask_and_select(logits + i * n_pad, n_pad, n_pad, tab);\n  }\n  free(y);"),
]


def _run_pins_against(source_text, tmp_path):
    mutant = tmp_path / "oracle_copy.c"
    mutant.write_text(source_text)
    so = tmp_path / "liboracle_copy.so"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                           str(so), str(mutant), "-lm"])
    env = dict(os.environ, EXL3_ORACLE_LIB_OVERRIDE=str(so), OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=600)


def test_control_unmutated_copy_passes_the_pins(tmp_path):
    """The harness itself: an unchanged copy built and loaded the same way
    passes every pin, so a failing mutant fails because of its mutation."""
    r = _run_pins_against(open(SRC).read(), tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


def test_mutations_apply_once():
    src = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1
    r = _run_pins_against(src.replace(old, new), tmp_path)
    assert r.returncode != 0, "mutation %s survived every pin:\n%s" % (name, r.stdout[-2000:])
