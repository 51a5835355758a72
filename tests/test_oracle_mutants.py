"""The pins must catch plausible mistakes in the oracle.

Each case compiles a copy of oracle.c with one planted mistake (on the CPU,
into a temporary directory) and runs the pin suite against it; the suite must
fail.  Mistakes that are provably equivalent (e.g. fmaf(s,q,b) vs s*q+b, equal
because s*q is exact for a bf16 s and a 4-bit q) are not listed.
"""
import os
import subprocess
import sys

import pytest

import oracle

MUTANTS = [
    ("nibble order reversed", "return (int)((w >> (4 * i)) & 0xFu);", "return (int)((w >> (28 - 4 * i)) & 0xFu);"),
    ("bias dropped", "return fmaf(orc_bf16_to_f32(s_bits), (float)q, orc_bf16_to_f32(b_bits));",
     "return orc_bf16_to_f32(s_bits) * (float)q;"),
    ("bias sign", "return fmaf(orc_bf16_to_f32(s_bits), (float)q, orc_bf16_to_f32(b_bits));",
     "return fmaf(orc_bf16_to_f32(s_bits), (float)q, -orc_bf16_to_f32(b_bits));"),
    ("group index uses 128", "int64_t g = k / G;", "int64_t g = k / 128;"),
    ("word index", "qw[n * (K / 8) + k / 8], (int)(k % 8));\n    int64_t g", "qw[n * (K / 8) + k % 8], (int)(k % 8));\n    int64_t g"),
    ("x transposed", "(double)orc_bf16_to_f32(x[m * K + k]) * w", "(double)orc_bf16_to_f32(x[k * M + m]) * w"),
    ("fp32 products", "double p = (double)orc_bf16_to_f32(x[m * K + k]) * w;",
     "double p = (double)(float)((double)orc_bf16_to_f32(x[m * K + k]) * w);"),
    ("bf16 double rounding", "double a = fabs(v);", "double a = fabs((double)(float)v);"),
    ("ties to the highest index", "if (y[n] > y[b])", "if (y[n] >= y[b])"),
    ("scale/bias swapped", "return orc_dequant(scales[n * (K / G) + g], biases[n * (K / G) + g], q);",
     "return orc_dequant(biases[n * (K / G) + g], scales[n * (K / G) + g], q);"),
    ("routed expert offset", "const uint32_t *qe = qw + e * N * (K / 8);", "const uint32_t *qe = qw + (E - 1 - e) * N * (K / 8);"),
    ("GELU by the tanh approximation", "double gelu = 0.5 * g * (1.0 + erf(g / sqrt(2.0)));",
     "double gelu = 0.5 * g * (1.0 + tanh(sqrt(2.0 / 3.141592653589793) * (g + 0.044715 * g * g * g)));"),
    ("GELU on the up rows", "h[i] = gelu * up[i];", "h[i] = 0.5 * up[i] * (1.0 + erf(up[i] / sqrt(2.0))) * g;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation anchor for '{name}' not unique"
    mut_c = tmp_path / "oracle_mutant.c"
    mut_c.write_text(src.replace(old, new))
    mut_so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(mut_so), str(mut_c), "-lm"], check=True)
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, W4A16_ORACLE_LIB=str(mut_so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(here, "test_oracle_pins.py")], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch '{name}':\n{r.stdout[-2000:]}"
