"""Plants plausible slips in copies of the CPU oracle and checks that the pins
in ``test_oracle_pins.py`` catch every one.  Runs on the CPU only: each mutant
is compiled with gcc into a temporary directory and loaded in place of the
real oracle for the duration of its check."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as P
import test_oracle_softmax_pins as S

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_gemm.c")

# (name, text in oracle_gemm.c, replacement).  Each text must occur exactly once.
MUTANTS = [
    ("strides swapped in the view decoder", "d[r * cols + c] = dec(base, r * sr + c * sc, dtype);",
     "d[r * cols + c] = dec(base, r * sc + c * sr, dtype);"),
    ("fp32 running sum", "acc[j] += a * brow[j];", "acc[j] = (float)(acc[j] + a * brow[j]);"),
    ("last k dropped", "for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k < K - 1; ++k) {"),
    ("B read transposed", "acc[j] += a * brow[j];", "acc[j] += a * Bd[j * K + k];"),
    ("A read transposed", "const double a = Ad[i * K + k];",
     "const double a = Ad[(k * M + i) % (M * K)];"),
    ("accumulator not reset per row", "acc[j] = 0.0;", "(void)0;"),
    ("output index transposed", "store(Cout, i * N + j, out_dtype, acc[j]);",
     "store(Cout, (j * M + i), out_dtype, acc[j]);"),
    ("f16 sign dropped", "v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */\n"
     "    return s ? -v : v;", "v = ldexp((double)(1024 + m), e - 25);\n    return v;"),
    ("f16 exponent bias off by one", "e - 25)", "e - 24)"),
    ("bf16 exponent bias off by one", "e - 134)", "e - 133)"),
    ("f16 subnormal scale wrong", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("ties away from zero", "double r = nearbyint(q);", "double r = round(q);"),
    ("truncating conversion", "double r = nearbyint(q);", "double r = floor(q);"),
    ("binade carry forgets the exponent", "n >>= 1;\n        e += 1;", "n >>= 1;"),
    ("no gradual underflow", "if (e < emin)\n        e = emin;", "if (0)\n        e = emin;"),
    ("overflow threshold off", "if (e > bias)\n", "if (e > bias + 1)\n"),
    ("fp16acc: partial not rounded", "const double p16 = dec_f16((uint16_t)rne(partial, 10, 5));",
     "const double p16 = partial;"),
    ("fp16acc: accumulator not rounded", "acc = dec_f16((uint16_t)rne(acc + p16, 10, 5));",
     "acc = acc + p16;"),
    ("fp16acc: chunk boundary off", "const int64_t k1 = k0 + BK < K ? k0 + BK : K;",
     "const int64_t k1 = k0 + BK + 1 < K ? k0 + BK + 1 : K;"),
    ("softmax: max not subtracted", "y[j] = exp(y[j] - m);", "y[j] = exp(y[j]);"),
    ("softmax: min instead of max", "if (x > m) /* false for NaN: the max ignores it */",
     "if (m == -INFINITY || x < m)"),
    ("softmax: last column left out of the sum", "sum += y[j];",
     "if (j + 1 < N) sum += y[j];"),
    ("softmax: strides swapped", "const double x = dec(X, i * sxm + j * sxn, in_dtype);",
     "const double x = dec(X, i * sxn + j * sxm, in_dtype);"),
    ("softmax: divides by the max term", "y[j] = y[j] / sum;", "y[j] = y[j] / exp(0.0);"),
    ("softmax: output row index", "store(Yout, i * N + j, out_dtype, y[j]);",
     "store(Yout, j * M + i < M * N ? j * M + i : 0, out_dtype, y[j]);"),
]

PINS = [
    P.test_worked_2x2,
    P.test_sentinel_table_correct,
    P.test_sentinel_nan_is_never_read,
    P.test_accumulation_seed0_fp32acc,
    P.test_accumulation_seed0_fp16acc,
    lambda: P.test_arange_closed_form_exact(33, 17, 65),
    lambda: P.test_integer_brute_force_vs_numpy_int64("f16", "f32"),
    lambda: P.test_integer_brute_force_vs_numpy_int64("bf16", "bf16"),
    lambda: P.test_integer_brute_force_vs_numpy_int64("f32", "f16"),
    P.test_strided_view_equals_contiguous_copy,
    P.test_fp64_sum_is_accurate,
    P.test_decode_f16_exhaustive,
    P.test_decode_bf16_exhaustive,
    P.test_encode_f16_and_f32_vs_numpy,
    P.test_encode_bf16,
    S.test_closed_forms,
    S.test_max_is_subtracted,
    S.test_special_values,
    S.test_rows_sum_to_one_and_match_scipy,
    S.test_strided_views,
    lambda: S.test_output_rounding_matches_numpy("f16"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _compile(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-w", "-shared",
                    "-fPIC", c, "-o", path, "-lm"], check=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, workdir):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    so = os.path.join(workdir, "m%d.so" % MUTANTS.index((name, old, new)))
    _compile(text.replace(old, new), so)
    saved = oracle._lib
    oracle._lib = oracle.load_library(so)
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, RuntimeError, ValueError, IndexError):
                caught.append(getattr(pin, "__name__", "lambda"))
                break
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught the mutant: {name}"
