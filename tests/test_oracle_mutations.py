"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (a wrong tie
rule, a dropped factor, a transposed index, a wrong constant, ...), builds it
on the CPU, and runs the pin suites against that build.  Every mutant must make
at least one pin fail.  Nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "w4a8_oracle.c")

MUTANTS = [
    ("integer scale rounded instead of ceil", "int64_t s = (D + 14) / 15;", "int64_t s = (D + 7) / 15;"),
    ("zero point truncated", "int64_t zz = orc_rne_div(-lo, s);", "int64_t zz = (-lo) / s;"),
    ("activation ties away from zero", "q = clampf(rintf(t), -127.0f, 127.0f);",
     "q = clampf(roundf(t), -127.0f, 127.0f);"),
    ("wrong protective range", "orc_f32_to_f16(a / (float)ORC_PROTECT)", "orc_f32_to_f16(a / 127.0f)"),
    ("zero not multiplied by the scale", "int64_t v = prod - zs;", "int64_t v = prod - zz;"),
    ("transposed weight index", "(int64_t)r[n * K + k];", "(int64_t)r[k * N + n];"),
    ("channel scale dropped", "t = t * orc_f16_to_f32(s0[n]);", "t = t * 1.0f;"),
    ("token scale dropped", "t = t * s_a[m];", "t = t * 1.0f;"),
    ("group range without zero", "int64_t lo = 0, hi = 0;", "int64_t lo = 127, hi = -128;"),
    ("integer ties always up", "q += (q & 1);", "q += 1;"),
    ("activation levels 128", "float s = a / 127.0f;", "float s = a / 128.0f;"),
    ("group index off by one", "int64_t s = s1[n * G + k / ORC_GROUP];",
     "int64_t s = s1[n * G + (k + 1) / ORC_GROUP % G];"),
    ("fp16 rounding truncates", "double n = rint(ldexp(a, 10 - e));", "double n = floor(ldexp(a, 10 - e));"),
    ("level-1 codes unclamped sign flip", "q8[n * K + k] = (int8_t)q;", "q8[n * K + k] = (int8_t)(-q);"),
    ("norm variance divisor K - 1", "double var = ss / (double)K;", "double var = ss / (double)(K - 1);"),
    ("norm eps dropped", "double ve = var + (double)eps;", "double ve = var;"),
    ("layernorm mean not subtracted", "float t = orc_f16_to_f32(xm[k]) - mean32;",
     "float t = orc_f16_to_f32(xm[k]);"),
    ("norm beta dropped", "t = t + orc_f16_to_f32(beta[k]);", "t = t + 0.0f;"),
    ("norm gamma index shifted", "t = t * orc_f16_to_f32(gamma[k]);",
     "t = t * orc_f16_to_f32(gamma[(k + 1) % K]);"),
    ("norm mean in single precision", "mean = ldexp((double)S, -24) / (double)K;",
     "mean = (double)(float)(ldexp((double)S, -24) / (double)K);"),
    ("norm rsqrt in single precision", "double r = ve == 0.0 ? INFINITY : 1.0 / sqrt(ve);",
     "double r = ve == 0.0 ? INFINITY : 1.0 / (double)sqrtf((float)ve);"),
    ("w4a16 weight index transposed", "(double)r[n * K + k] * sc;", "(double)r[(k * N + n) % (N * K)] * sc;"),
    ("w4a16 channel scale dropped", "const double sc = (double)orc_f16_to_f32(s0[n]);", "const double sc = 1.0;"),
    ("w4a16 products in single precision",
     "const double p = (double)orc_f16_to_f32(x[m * K + k]) * (double)r[n * K + k] * sc;",
     "const double p = (double)(orc_f16_to_f32(x[m * K + k]) * (float)r[n * K + k] * (float)sc);"),
    ("kv range without zero", "float lo = 0.0f, hi = 0.0f;\n        for (int64_t d = 0; d < D; d++) {\n            const float v",
     "float lo = INFINITY, hi = -INFINITY;\n        for (int64_t d = 0; d < D; d++) {\n            const float v"),
    ("kv sixteen levels", "orc_f32_to_f16((hi - lo) / 15.0f)", "orc_f32_to_f16((hi - lo) / 16.0f)"),
    ("kv zero point truncated", "clampf(rintf(-lo / sf), 0.0f, 15.0f)", "clampf(truncf(-lo / sf), 0.0f, 15.0f)"),
    ("kv code ties away from zero", "rintf(orc_f16_to_f32(xi[d]) / sf) + zf", "roundf(orc_f16_to_f32(xi[d]) / sf) + zf"),
    ("kv key zero not subtracted", "((double)kc[(row0 + t) * D + d] - (double)kz[row0 + t]) * kscale",
     "((double)kc[(row0 + t) * D + d]) * kscale"),
    ("kv value zero added", "((double)vc[(row0 + t) * D + d] - (double)vz[row0 + t]) * vscale",
     "((double)vc[(row0 + t) * D + d] + (double)vz[row0 + t]) * vscale"),
    ("kv head modulo instead of group", "const int64_t g = h / G;", "const int64_t g = h % Hkv;"),
    ("attention scale dropped", "sc[t] = sm_scale * dot;", "sc[t] = dot;"),
    ("softmax normalizer without the max", "den = den + exp(sc[t] - mx);", "den = den + exp(sc[t]);"),
    ("value scale taken from the keys", "const double vscale = (double)orc_f16_to_f32(vs[row0 + t]);",
     "const double vscale = (double)orc_f16_to_f32(ks[row0 + t]);"),
    ("attention length off by one", "for (int64_t t = 0; t < L; t++) {\n                const double kscale",
     "for (int64_t t = 0; t <= L && t < S; t++) {\n                const double kscale"),
]
PIN_FILES = ["test_oracle_pins.py", "test_oracle_norm_pins.py", "test_oracle_w4a16_pins.py",
             "test_oracle_kv4_pins.py"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: %s" % old
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(lib), str(mutant), "-lm"], check=True)
    env = dict(os.environ, W4A8_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"]
                         + [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, "mutant '%s' passed every pin:\n%s" % (name, res.stdout[-2000:])
