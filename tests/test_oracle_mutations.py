"""Plants plausible mistakes in a copy of the CPU oracle and checks that the
pins in test_oracle_pins.py catch every one (CPU only; mutants are compiled
into a temporary directory and never touch the real oracle)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "gate_up_swapped": ("matvec(w13, wdt, s13, 0, I, H, xv, rowbuf, g);\n    matvec(w13, wdt, s13, I, I, H, xv, rowbuf, u);",
                        "matvec(w13, wdt, s13, I, I, H, xv, rowbuf, g);\n    matvec(w13, wdt, s13, 0, I, H, xv, rowbuf, u);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "ties_to_high_id": ("(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    "no_renormalise": ("w[t * K + j] = p[ids[t * K + j]] / s;", "w[t * K + j] = p[ids[t * K + j]];"),
    "shared_dropped": ("out[t * H + h] = acc + (s ? s[t * H + h] : 0.0);", "out[t * H + h] = acc;"),
    "padding_off_by_one": ("((mode == 1 ? maxn : counts[e]) + B - 1) / B * B",
                           "((mode == 1 ? maxn : counts[e]) + B) / B * B"),
    "max_padding_uses_own_count": ("(mode == 1 ? maxn : counts[e])", "(counts[e])"),
    "bucket_descending": ("int64_t r = offsets[e] + fill[e];",
                          "int64_t r = offsets[e] + (counts[e] - 1 - fill[e]);"),
    "wrong_expert_weights": ("(size_t)ids[k] * 2 * I * H * esize", "(size_t)ids[(k + 1) % K] * 2 * I * H * esize"),
    "combine_slot_mixup": ("acc += w[t * K + k] * y[(t * K + k) * H + h];",
                           "acc += w[t * K + (K - 1 - k)] * y[(t * K + k) * H + h];"),
    "down_proj_transposed": ("matvec(w2, wdt, s2, 0, H, I, a, rowbuf, y);",
                             "for (int hh = 0; hh < H; ++hh) { double s2 = 0; for (int i = 0; i < I; ++i) "
                             "s2 += elem(w2, wdt, (int64_t)i * H + hh) * a[i]; y[hh] = s2; }"),
    "fp8_exponent_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    "fp8_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "fp8_row_scale_ignored": ("const double sc = scale ? (double)scale[row] : 1.0;",
                              "const double sc = 1.0;"),
    "budget_renormalised_over_kmax": ("orc_route(logits + t * E, 1, E, k, ids + t * Kmax, w + t * Kmax)",
                                      "orc_route(logits + t * E, 1, E, Kmax, ids + t * Kmax, w + t * Kmax)"),
    "unused_slot_counted": ("if (ids[p] >= 0)\n            counts[ids[p]] += 1;",
                            "counts[ids[p] < 0 ? 0 : ids[p]] += 1;"),
    "layer_ignores_budget": ("const int32_t kt = k_tok ? k_tok[t] : K;", "const int32_t kt = K;"),
    "combine_reads_unused_rows": ("if (w[t * K + k] != 0.0)", "if (1)"),
    "block_map_overrun": ("for (int64_t b = offsets[e] / B; b < offsets[e + 1] / B; ++b)",
                          "for (int64_t b = offsets[e] / B; b <= offsets[e + 1] / B && b < cap / B; ++b)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, "mutation site moved; update the mutant"
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(c), "-o",
                           str(so), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 1, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
