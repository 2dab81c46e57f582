"""The oracle's pins must catch plausible mistakes.

Each case plants one slip in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the fast pin tests against
that copy in a subprocess: every mutant must make them fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tg_oracle.c")

MUTANTS = {
    "dropped_last_k_term": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {"),
    "reversed_k_in_A": ("decode(dtype, A[i * K + k])", "decode(dtype, A[i * K + (K - 1 - k)])"),
    "bias_after_gelu": ("y = y + biasd[j];\n            if (epilogue == OR_EPI_BIAS_GELU_TANH)\n                y = gelu_tanh(y);",
                        "if (epilogue == OR_EPI_BIAS_GELU_TANH)\n                y = gelu_tanh(y);\n            y = y + biasd[j];"),
    "erf_gelu": ("return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));",
                 "(void)c; return 0.5 * y * (1.0 + erf(y / sqrt(2.0)));"),
    "ties_away_from_zero": ("double n = nearbyint(", "double n = round("),
    "f16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "bf16_exponent_bias": ("v = ldexp((double)(f + 128), e - 134);", "v = ldexp((double)(f + 128), e - 133);"),
    "gelu_constant": ("0.044715 * y * y * y", "0.04715 * y * y * y"),
    "w4_zero_point": ("((double)Q[k * N + j] - 8.0)", "((double)Q[k * N + j] - 7.0)"),
    "w4_q_transposed": ("((double)Q[k * N + j] - 8.0)", "((double)Q[j * K + k] - 8.0)"),
    "w4_scale_group_shift": ("scales[(k / group) * N + j]", "scales[((k / group + 1) % (K / group)) * N + j]"),
    "w4_scale_transposed": ("scales[(k / group) * N + j]", "scales[j * (K / group) + k / group]"),
    "w4_sign": ("((double)Q[k * N + j] - 8.0) *", "(8.0 - (double)Q[k * N + j]) *"),
    "attn_no_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "attn_causal_strict": ("const int64_t nk = causal ? i + 1 : Sk;", "const int64_t nk = causal ? i : Sk;"),
    "attn_no_max": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "attn_bhsd_keys": ("const uint16_t *krow = K + ((b * Sk + j) * H + h) * D;",
                       "const uint16_t *krow = K + ((b * H + h) * Sk + j) * D;"),
    "attn_bhsd_values": ("const uint16_t *vrow = V + ((b * Sk + j) * H + h) * D;",
                         "const uint16_t *vrow = V + ((b * H + h) * Sk + j) * D;"),
    "attn_unnormalized": ("o[d] = nk > 0 ? o[d] / l : 0.0;", "o[d] = nk > 0 ? o[d] : 0.0;"),
}

FAST_PINS = ["tests/test_oracle_codec.py", "tests/test_oracle_gemm.py", "tests/test_oracle_w4.py",
             "tests/test_oracle_attention.py",
             "-k", "not workload_shapes and not blas and not thread_count"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(lib), str(mutant_c), "-lm"], check=True)
    env = dict(os.environ, TG_ORACLE_LIBRARY=str(lib), PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *FAST_PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
