"""Mutation check of the oracle's pins: plant one plausible mistake at a time
in a copy of oracle.c (on the CPU), build it, and require that the pin suite
fails against it.  Each mutant runs in its own process, so a mutant that
crashes also counts as caught.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text to find, replacement) — each text must occur in oracle.c.
MUTANTS = [
    ("f16 exponent bias off by one", "ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    ("f16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("bf16 exponent bias", "ldexp((double)(128 + m), e - 134)", "ldexp((double)(128 + m), e - 133)"),
    ("f32 implicit bit dropped", "ldexp((double)(8388608u + m), e - 150)", "ldexp((double)(m), e - 150)"),
    ("int8 sign bit weight", "((s[i] & 0x80) ? 128.0 : 0.0)", "((s[i] & 0x80) ? 127.0 : 0.0)"),
    ("int32 read as unsigned", "((s[i] & 0x80000000u) ? 2147483648.0 : 0.0)",
     "((s[i] & 0x80000000u) ? -2147483648.0 : 0.0)"),
    ("leaky slope dropped", "return z >= 0.0 ? z : alpha * z;", "return z >= 0.0 ? z : z;"),
    ("leaky branches swapped", "return z >= 0.0 ? z : alpha * z;", "return z >= 0.0 ? alpha * z : z;"),
    ("relu keeps negatives", "return z > 0.0 ? z : 0.0;", "return z > 0.0 ? z : -z;"),
    ("tanh dropped", "return tanh(z);", "return z;"),
    ("gelu erfc argument unscaled", "return z * 0.5 * erfc(-z / sqrt(2.0));",
     "return z * 0.5 * erfc(-z);"),
    ("gelu tanh approximation", "return z * 0.5 * erfc(-z / sqrt(2.0));",
     "return z * 0.5 * (1.0 + tanh(sqrt(2.0 / 3.141592653589793) * (z + 0.044715 * z * z * z)));"),
    ("gelu cdf of -z", "return z * 0.5 * erfc(-z / sqrt(2.0));",
     "return z * 0.5 * erfc(z / sqrt(2.0));"),
    ("gelu via 1 + erf (cancels in the tail)", "return z * 0.5 * erfc(-z / sqrt(2.0));",
     "return z * 0.5 * (1.0 + erf(z / sqrt(2.0)));"),
    ("residual dropped", "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i] + r[i], alpha);",
     "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i], alpha);"),
    ("residual after the activation", "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i] + r[i], alpha);",
     "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i], alpha) + r[i];"),
    ("residual subtracted", "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i] + r[i], alpha);",
     "for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i] - r[i], alpha);"),
    ("sigmoid sign", "if (z >= 0.0) return 1.0 / (1.0 + exp(-z));", "if (z >= 0.0) return 1.0 / (1.0 + exp(z));"),
    ("sigmoid negative branch", "return exp(z) / (1.0 + exp(z));", "return 1.0 / (1.0 + exp(z));"),
    ("gemm bias dropped", "double z = acc[j] + (bias ? bias[j] : 0.0);", "double z = acc[j];"),
    ("gemm bias indexed by row", "double z = acc[j] + (bias ? bias[j] : 0.0);",
     "double z = acc[j] + (bias ? bias[i % N] : 0.0);"),
    ("gemm B read transposed", "const double *brow = B + k * N;", "const double *brow = B + (k % N) * N;"),
    ("gemm first k skipped", "for (int64_t k = 0; k < K; ++k) {\n                    double a",
     "for (int64_t k = 1; k < K; ++k) {\n                    double a"),
    ("conv pad sign", "int64_t iw = ow * s->sw - s->pl + q * s->dw;", "int64_t iw = ow * s->sw + s->pl + q * s->dw;"),
    ("conv pads top/left swapped", "s->pt = pads[0]; s->pb = pads[1]; s->pl = pads[2]; s->pr = pads[3];",
     "s->pt = pads[0]; s->pb = pads[2]; s->pl = pads[1]; s->pr = pads[3];"),
    ("conv dilation dropped", "int64_t ih = oh * s->sh - s->pt + r * s->dh;", "int64_t ih = oh * s->sh - s->pt + r;"),
    ("conv stride dropped", "int64_t ih = oh * s->sh - s->pt + r * s->dh;", "int64_t ih = oh - s->pt + r * s->dh;"),
    ("conv kernel flipped", "w[((co * s->C + c) * s->kh + r) * s->kw + q]",
     "w[((co * s->C + c) * s->kh + (s->kh - 1 - r)) * s->kw + (s->kw - 1 - q)]"),
    ("conv channel index of w", "w[((co * s->C + c) * s->kh + r) * s->kw + q]",
     "w[((co * s->C + (s->C - 1 - c)) * s->kh + r) * s->kw + q]"),
    ("conv bias dropped", "return acc + (bias ? bias[co] : 0.0);", "return acc;"),
    ("conv out size rounds up", "return span / stride + 1;", "return (span + stride - 1) / stride + 1;"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, find, repl, tmp_path):
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutation site not found: {find!r}"
    msrc = tmp_path / "oracle.c"
    msrc.write_text(src.replace(find, repl))
    # the header sits next to the original source
    lib = str(tmp_path / "liboracle_mut.so")
    orc.build(src=str(msrc), out=lib, extra_flags=["-I", os.path.dirname(SRC)])
    env = dict(os.environ, BIASACT_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant '{name}' survived the pins:\n{r.stdout[-2000:]}"
