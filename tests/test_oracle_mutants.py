"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source (a dropped term, a wrong sign or index, a transposed
operand, a broken order or rounding) makes the pin suite fail. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
T = os.path.join(ROOT, "tests")

MUTANTS = [
    # (name, original text, planted mistake, pin files that must catch it)
    ("silu_sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))", ["test_oracle_ffn.py"]),
    ("down_transposed", "wo + (size_t)j * d + c", "wo + (size_t)c * f + j", ["test_oracle_ffn.py"]),
    ("router_weight_dropped", "acc[c] += wk * y[c];", "acc[c] += y[c];", ["test_oracle_ffn.py"]),
    ("gate_up_swapped", "h[j] = silu(g[j]) * u[j];", "h[j] = silu(u[j]) * g[j];", ["test_oracle_ffn.py"]),
    ("h_not_rounded", "h[j] = round_to(h[j], dtype);", "h[j] = h[j];", ["test_oracle_ffn.py"]),
    ("pad_off_by_one", "((int64_t)cnt[e] + tm - 1) / tm * tm", "((int64_t)cnt[e] + tm) / tm * tm",
     ["test_oracle_plan.py"]),
    ("placement_not_stable", "for (int64_t i = 0; i < nent; ++i) {\n        int e = ids[i];\n        if (e < 0 || e >= E) {",
     "for (int64_t i = nent - 1; i >= 0; --i) {\n        int e = ids[i];\n        if (e < 0 || e >= E) {",
     ["test_oracle_plan.py"]),
    ("skip_counted_as_bad", "if (e == -1)\n            nskip++;", "if (e == -2)\n            nskip++;",
     ["test_oracle_plan.py"]),
    ("gather_pad_not_zero", "memset(dst, 0, rb);", "(void)dst;", ["test_oracle_gather_combine.py"]),
    ("combine_reversed",
     "for (int k = 0; k < K; ++k) {\n                int32_t r = pos[t * K + k];\n                if (r >= 0)\n                    acc = acc + Y[",
     "for (int k = K - 1; k >= 0; --k) {\n                int32_t r = pos[t * K + k];\n                if (r >= 0)\n                    acc = acc + Y[",
     ["test_oracle_gather_combine.py"]),
    ("f16_truncates", "double q = nearbyint(ldexp(a, 10 - E));", "double q = floor(ldexp(a, 10 - E));",
     ["test_oracle_formats.py"]),
    ("bf16_subnormal_flush", "double q = nearbyint(ldexp(a, 133));", "double q = 0.0 * a;",
     ["test_oracle_formats.py"]),
    ("y16_exponent_off_by_one", "int e = 15 - k;", "int e = 16 - k;", ["test_oracle_y16.py"]),
    ("y16_decode_wrong_sign", "y[(size_t)r * d + c] = (float)ldexp(oracle_f16_to_f64(s[(size_t)r * d + c]),\n                                                -(int)ex[",
     "y[(size_t)r * d + c] = (float)ldexp(oracle_f16_to_f64(s[(size_t)r * d + c]),\n                                                +(int)ex[",
     ["test_oracle_y16.py"]),
    ("combine_y16_block_index", "-(int)ex[(size_t)r * nb + c / Y16_BLOCK]);\n            }",
     "-(int)ex[(size_t)r * nb + c % nb]);\n            }", ["test_oracle_y16.py"]),
]


@pytest.mark.parametrize("name,old,new,files", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, files):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(mut), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + [os.path.join(T, f) for f in files],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' was not caught:\n{r.stdout[-2000:]}"
