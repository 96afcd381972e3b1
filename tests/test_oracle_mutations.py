"""The oracle's pins are sensitive: each planted mistake makes at least one pin fail.

Every case copies ``oracle/ssq_oracle.c``, plants one plausible mistake in the
copy (a dropped term, a wrong sign, a wrong index, an off-by-one grid, a
swapped readout ...), builds it with gcc into a temporary directory, points
the oracle binding at it and runs every test of ``test_oracle_pins``.  The
case passes only if some pin fails.  Nothing here touches a GPU.
"""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins
from tests import test_oracle_sr as sr_pins
from tests import test_oracle_kda as kda_pins
from tests import test_oracle_prefill as prefill_pins
from tests import test_oracle_damp as damp_pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "ssq_oracle.c")).read()

# (name, text in ssq_oracle.c, replacement); the text must occur exactly `count` times
MUTATIONS = [
    ("fp32 write term dropped", "            float wb = w * Bn[n];\n            h[n] = fmaf(lam, h[n], wb);",
     "            float wb = 0.0f * Bn[n];\n            h[n] = fmaf(lam, h[n], wb);"),
    ("quantized write term dropped",
     "        float wb = w * Bn[n];\n        work[n] = fmaf(lam, work[n], wb);",
     "        float wb = 0.0f * Bn[n];\n        work[n] = fmaf(lam, work[n], wb);"),
    ("quantized update in the fused order (decay on the scale, offset in the write term)",
     "    orc_dequantize_row(code, N, *s, *z, work);\n    for (n = 0; n < N; ++n) {\n"
     "        float wb = w * Bn[n];\n        work[n] = fmaf(lam, work[n], wb);",
     "    for (n = 0; n < N; ++n) {\n        float ls = lam * (*s);\n"
     "        float wb = fmaf(w, Bn[n], -(ls * (*z)));\n        work[n] = fmaf(ls, (float)code[n], wb);"),
    ("quantized update rounds the decayed term", "        work[n] = fmaf(lam, work[n], wb);",
     "        work[n] = lam * work[n] + wb;"),
    ("zero point added instead of subtracted", "        float d = (float)code[i] - z;",
     "        float d = (float)code[i] + z;"),
    ("zero point dropped in reconstruction", "        float d = (float)code[i] - z;",
     "        float d = (float)code[i];"),
    ("zero point sign flipped", "float z = (float)(-rne_sum((double)mn * (double)inv, 0.0)) + 0.0f;",
     "float z = (float)(rne_sum((double)mn * (double)inv, 0.0)) + 0.0f;"),
    ("zero point from the max", "float z = (float)(-rne_sum((double)mn * (double)inv, 0.0)) + 0.0f;",
     "float z = (float)(-rne_sum((double)mx * (double)inv, 0.0)) + 0.0f;"),
    ("symmetric grid off by one", "const float cmax = (float)((1 << (bits - 1)) - 1);",
     "const float cmax = (float)((1 << (bits - 1)));"),
    ("asymmetric grid off by one", "const float cmax = (float)((1 << bits) - 1);",
     "const float cmax = (float)((1 << bits));"),
    ("Euler decay instead of exp", "return (float)exp((double)e);", "return (float)(1.0 + (double)e);"),
    ("decay applied twice", "        work[n] = fmaf(lam, work[n], wb);", "        work[n] = fmaf(lam * lam, work[n], wb);"),
    ("readouts swapped", "    if (readout_pre) {\n        for (n = 0; n < N; ++n)",
     "    if (!readout_pre) {\n        for (n = 0; n < N; ++n)"),
    ("D*x dropped", "float dx = D * x;", "float dx = 0.0f * x;"),
    ("ties always up", "k = (fmod(f + z, 2.0) == 0.0) ? f : f + 1.0;", "k = f + 1.0;"),
    ("rounding to the floor", "    if (r > 0.5)\n        k = f + 1.0;", "    if (r > 1.5)\n        k = f + 1.0;"),
    ("top clamp missing", "            if (t > (double)cmax)\n                t = (double)cmax;\n            code[i] = (int32_t)t;\n            if (v_out)\n                v_out[i] = v;\n        }\n        *s_out = s;\n        *z_out = z;",
     "            code[i] = (int32_t)t;\n            if (v_out)\n                v_out[i] = v;\n        }\n        *s_out = s;\n        *z_out = z;"),
    ("scan reads token 0 every step", "memcpy(xs + (size_t)b * H * P, x + ((size_t)b * T + t) * H * P",
     "memcpy(xs + (size_t)b * H * P, x + ((size_t)b * T + 0) * H * P"),
    ("group index wrong", "            int g = hh / (H / G);\n            const float *Bn = Bm + ((int64_t)b * G + g) * N;",
     "            int g = hh % G;\n            const float *Bn = Bm + ((int64_t)b * G + g) * N;"),
    ("prefill group index wrong", "            int g = hh / (H / G);\n            for (p = 0; p < P; ++p) {",
     "            int g = hh % G;\n            for (p = 0; p < P; ++p) {"),
    ("delta correction sign", "            vm = v[j] - au;", "            vm = v[j] + au;"),
    ("delta decay not applied to the state", "Sn[(int64_t)i * dv + j] = fmaf(al, Sh[(int64_t)i * dv + j], kw);",
     "Sn[(int64_t)i * dv + j] = Sh[(int64_t)i * dv + j] + kw;"),
    ("delta state reconstructed without its scale",
     "            orc_dequantize_row(code + (int64_t)i * dv, dv, s[i], z[i], Sh + (int64_t)i * dv);",
     "            orc_dequantize_row(code + (int64_t)i * dv, dv, 1.0f, z[i], Sh + (int64_t)i * dv);"),
    ("delta update in the fused order",
     "            float kw = k[i] * w[j];\n            Sn[(int64_t)i * dv + j] = fmaf(al, Sh[(int64_t)i * dv + j], kw);",
     "            float kw = bits ? fmaf(k[i], w[j], -((al * s[i]) * z[i])) : k[i] * w[j];\n"
     "            Sn[(int64_t)i * dv + j] = bits ? fmaf(al * s[i], (float)code[(int64_t)i * dv + j], kw)\n"
     "                                           : fmaf(al, Sh[(int64_t)i * dv + j], kw);"),
    ("two-tier uint8 rows updated in the fused order",
     "                float kw = km[i] * wt[j];\n                St[(int64_t)i * dv + j] = fmaf(al, Sh[(int64_t)i * dv + j], kw);",
     "                float kw = i < nhi ? km[i] * wt[j] : fmaf(km[i], wt[j], -((al * sm[i - nhi]) * zm[i - nhi]));\n"
     "                St[(int64_t)i * dv + j] = i < nhi ? fmaf(al, Sh[(int64_t)i * dv + j], kw)\n"
     "                    : fmaf(al * sm[i - nhi], (float)cm[(int64_t)(i - nhi) * dv + j], kw);"),
    ("delta readout with k instead of q",
     "                for (j = 0; j < dv; ++j)\n                    acc[j] += (double)q[i] * (double)Sn[(int64_t)i * dv + j];\n            }\n        }",
     "                for (j = 0; j < dv; ++j)\n                    acc[j] += (double)k[i] * (double)Sn[(int64_t)i * dv + j];\n            }\n        }"),
    ("delta u uses the wrong key index",
     "double kd = avec ? (double)k[i] * (double)avec[i] : (double)k[i];",
     "double kd = avec ? (double)k[i] * (double)avec[i] : (double)k[j % dk];"),
    ("dequantization scale dropped", "        out[i] = s * d;", "        out[i] = d;"),
    ("stochastic rounding rounds up below the threshold",
     "return f + z + (t + K >= 65536.0 ? 1.0 : 0.0);", "return f + z + (t + K > 65536.0 ? 1.0 : 0.0);"),
    ("stochastic rounding drops the zero point",
     "return f + z + (t + K >= 65536.0 ? 1.0 : 0.0);", "return f + (t + K >= 65536.0 ? 1.0 : 0.0);"),
    ("stochastic rounding compares U with the fraction, not 1 - U",
     "return f + z + (t + K >= 65536.0 ? 1.0 : 0.0);", "return f + z + (K > t ? 1.0 : 0.0);"),
    ("stochastic rounding takes the fraction from the rounded sum",
     "double t = floor(p * 65536.0) - f * 65536.0;", "double t = floor((p - f) * 65536.0);"),
    ("uniform counter ignores the token",
     "uint64_t ctr = (step * (uint64_t)rows + (uint64_t)r) * (uint64_t)N + (uint64_t)n;",
     "uint64_t ctr = ((uint64_t)r) * (uint64_t)N + (uint64_t)n;"),
    ("uniform pieces taken high first", "uint32_t K = (uint32_t)(out >> (16 * (ctr % 4))) & 0xFFFFu;",
     "uint32_t K = (uint32_t)(out >> (16 * (3 - ctr % 4))) & 0xFFFFu;"),
    ("one output per uniform", "uint64_t out = orc_splitmix64(seed, ctr / 4 + 1);",
     "uint64_t out = orc_splitmix64(seed, ctr + 1);"),
    ("scan reuses the first token's uniforms", "ys, readout_pre, NULL, NULL, sr, seed, step + (uint64_t)t);",
     "ys, readout_pre, NULL, NULL, sr, seed, step);"),
    ("delta draws the uniforms of the matrix's first row",
     "/* key row i of matrix m is state row m*dk + i */\n            for (i = 0; i < dk; ++i)\n"
     "                orc_sr_row_uniforms(seed, step, nm * dk, m * dk + i, dv, U + i * dv);",
     "/* key row i of matrix m is state row m*dk + i */\n            for (i = 0; i < dk; ++i)\n"
     "                orc_sr_row_uniforms(seed, step, nm * dk, m * dk, dv, U + i * dv);"),
    ("KDA decay missing from u", "double kd = avec ? (double)k[i] * (double)avec[i] : (double)k[i];",
     "double kd = (double)k[i];"),
    ("KDA decays every row with the first channel's gate", "float al = avec ? avec[i] : alpha;",
     "float al = avec ? avec[0] : alpha;"),
    ("KDA applies the decay to u twice", "            vm = v[j] - u[j];",
     "            vm = v[j] - avec[0] * u[j];"),
    ("prefill quantizes every token", "int end = ((t + 1) % chunk == 0) || t == T - 1;", "int end = 1;"),
    ("prefill ignores the chunk length", "int end = ((t + 1) % chunk == 0) || t == T - 1;",
     "int end = t == T - 1;"),
    ("prefill reads the fp32 state at a chunk end", "if (!end || readout_pre)", "if (1)"),
    ("prefill continues from the unrounded row",
     "sr ? U : NULL);\n                        orc_dequantize_row(c, N, s[row], z[row], r);",
     "sr ? U : NULL);"),
    ("chunk-end uniforms of the first token", "orc_sr_row_uniforms(seed, step + (uint64_t)t, rows, row, N, U);",
     "orc_sr_row_uniforms(seed, step, rows, row, N, U);"),
    ("Hadamard sign from the wrong bit", "return (c & 1) ? -1.0 / 16.0 : 1.0 / 16.0;",
     "return (c & 2) ? -1.0 / 16.0 : 1.0 / 16.0;"),
    ("v not rotated", "a += hs(j, i) * (double)vm[i];", "a += (i == j ? 1.0 : 0.0) * (double)vm[i];"),
    ("o not rotated back", "o[m * dv + j] = (float)(2.0 * a);", "o[m * dv + j] = (float)ot[j];"),
    ("half tier keeps the unrounded value", "him[(int64_t)i * dv + j] = orc_round_half(row[j]);",
     "him[(int64_t)i * dv + j] = row[j];"),
    ("half rounding ties away from zero", "r = rint((double)x / q) * q;", "r = round((double)x / q) * q;"),
    ("two-tier u ignores the half rows",
     "                memcpy(Sh + (int64_t)i * dv, him + (int64_t)i * dv, sizeof(float) * (size_t)dv);",
     "                memset(Sh + (int64_t)i * dv, 0, sizeof(float) * (size_t)dv);"),
]


def _pin_cases():
    cases = []
    members = []
    for mod in (pins, sr_pins, kda_pins, prefill_pins, damp_pins):
        members += inspect.getmembers(mod, inspect.isfunction)
    for name, fn in members:
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        grids = [m.args for m in marks if m.name == "parametrize"]
        combos = [dict()]
        for argnames, values in grids:
            names = [a.strip() for a in argnames.split(",")]
            new = []
            for c in combos:
                for v in values:
                    vv = v if len(names) > 1 else (v,)
                    new.append({**c, **dict(zip(names, vv))})
            combos = new
        for c in combos:
            cases.append((name, fn, c))
    return cases


def _failing_pins(lib_path):
    saved = oracle._lib
    oracle._lib = oracle.bind(lib_path)
    failed = []
    try:
        for name, fn, kw in _pin_cases():
            try:
                fn(**kw)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(name)
    finally:
        oracle._lib = saved
    return failed


def test_unmutated_copy_passes_every_pin(tmp_path):
    path = tmp_path / "liboracle_copy.so"
    src = tmp_path / "copy.c"
    src.write_text(SRC)
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(path), "-lm"])
    assert _failing_pins(str(path)) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation site for '{name}' not unique"
    src = tmp_path / "mut.c"
    src.write_text(SRC.replace(old, new))
    path = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(path), "-lm"])
    failed = _failing_pins(str(path))
    assert failed, f"no pin caught: {name}"
