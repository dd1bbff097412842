"""The oracle's pins catch plausible mistakes (mutation test, CPU only).

Each mutant below is a copy of ``oracle/nvfp4_oracle.c`` with one plausible
mistake planted in it: a wrong constant, index, sign, rounding rule, loop
bound or operand.  Each copy is compiled with the oracle's own flags.  The
oracle pin files then run against it in a child pytest process, which loads
the copy through ``NVFP4_ORACLE_LIB``.  Every mutant must make at least one
pin fail.  The unmutated source, built the same way, must pass them all,
which shows the harness itself works.  Nothing here touches the GPU path.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
HDR = os.path.join(ROOT, "oracle", "nvfp4_oracle.h")
# fastest first: a child stops at its first failing pin
PIN_FILES = ["tests/test_oracle_quant.py", "tests/test_oracle_gemm.py", "tests/test_oracle_rng.py",
             "tests/test_oracle_mx.py", "tests/test_oracle_codecs.py"]

# (name, text in the source, replacement); each text occurs exactly once
MUTANTS = [
    # format codecs
    ("e2m1 table: largest magnitude 5", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}",
     "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}"),
    ("e4m3 decode: exponent bias 8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3 decode: subnormal step 2^-10", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("e4m3 encode: ties to the odd byte", "(d == best_d && (b % 2) == 0)", "(d == best_d && (b % 2) == 1)"),
    ("e4m3 encode: 448 left out of the search", "for (int b = 1; b <= 0x7E; ++b)",
     "for (int b = 1; b < 0x7E; ++b)"),
    ("e2m1 rne: ties to the odd code", "(d == best_d && (i % 2) == 0)", "(d == best_d && (i % 2) == 1)"),
    ("e2m1 rne: sign of zero dropped",
     "  return (signbit(y) ? 8 : 0) | idx;\n}\n\n/* R5",
     "  return ((y < 0.0f) ? 8 : 0) | idx;\n}\n\n/* R5"),
    ("sr: rounds up when u equals the fraction", "((double)u16 < f * 65536.0)", "((double)u16 <= f * 65536.0)"),
    ("sr: fraction over hi instead of hi - lo", "(m - kE2M1[lo]) / (kE2M1[lo + 1] - kE2M1[lo])",
     "(m - kE2M1[lo]) / kE2M1[lo + 1]"),
    ("sr: saturation threshold 4", "  if (m >= 6.0) {\n    idx = 7;\n  } else {\n    int lo = 0;",
     "  if (m >= 4.0) {\n    idx = 7;\n  } else {\n    int lo = 0;"),
    # Philox and the draw layout
    ("philox: wrong first multiplier", "0xD2511F53u * c[0]", "0xD2511F55u * c[0]"),
    ("philox: high halves swapped", "uint32_t n0 = hi1 ^ c[1] ^ k[0];", "uint32_t n0 = hi0 ^ c[1] ^ k[0];"),
    ("philox: nine rounds", "for (int r = 0; r < 10; ++r)", "for (int r = 0; r < 9; ++r)"),
    ("philox: second Weyl increment", "k[1] += 0xBB67AE85u;", "k[1] += 0x9E3779B9u;"),
    ("draws: halves of a word swapped", "return (index & 1) ? (word >> 16) : (word & 0xFFFFu);",
     "return (index & 1) ? (word & 0xFFFFu) : (word >> 16);"),
    ("draws: stream in counter word 3", "{(uint32_t)g, (uint32_t)(g >> 32), stream, 0u}",
     "{(uint32_t)g, (uint32_t)(g >> 32), 0u, stream}"),
    ("draws: four elements per counter", "const uint64_t g = index >> 3;", "const uint64_t g = index >> 2;"),
    # transform
    ("rht: sign mask from stream 1", "const uint32_t ctr[4] = {0u, 0u, 2u, 0u};",
     "const uint32_t ctr[4] = {0u, 0u, 1u, 0u};"),
    ("rht: scale 1/2 instead of 1/4", "v[j] = 0.25f * v[j];", "v[j] = 0.5f * v[j];"),
    ("rht: last butterfly stage missing", "for (int h = 1; h < 16; h <<= 1)", "for (int h = 1; h < 8; h <<= 1)"),
    ("rht: signs applied to the wrong elements", "if ((sign_mask >> j) & 1u) v[j] = -v[j];",
     "if ((sign_mask >> (15 - j)) & 1u) v[j] = -v[j];"),
    # scales
    ("tensor scale: 448 / amax", "float s = 2688.0f / amax;", "float s = 448.0f / amax;"),
    ("tensor scale: zero amax gives 0", "if (amax == 0.0f) return 1.0f;", "if (amax == 0.0f) return 0.0f;"),
    ("tensor amax: signed maximum", "const float a = fabsf(v[i]);", "const float a = v[i];"),
    ("block scale: amax / 4", "const float s = t / 6.0f;", "const float s = t / 4.0f;"),
    ("block scale: other rounding order", "const float t = amax_b * s_enc;\n  const float s = t / 6.0f;",
     "const float t = s_enc / 6.0f;\n  const float s = amax_b * t;"),
    ("multiplier: tensor scale dropped", "float q = s_enc / sb;", "float q = 1.0f / sb;"),
    ("element: one ulp off", "const float y = x * inv;", "const float y = (x * inv) * 1.00000012f;"),
    ("input: bf16 widened one bit short", "(uint32_t)((const uint16_t*)x)[i] << 16",
     "(uint32_t)((const uint16_t*)x)[i] << 15"),
    # layouts
    ("columnwise: rowwise draw index", "seed, 1u, (uint64_t)(c * rows + r))", "seed, 1u, (uint64_t)(r * cols + c))"),
    ("columnwise: stream 0", "encode(v[r * cols + c], inv, rounding, seed, 1u,",
     "encode(v[r * cols + c], inv, rounding, seed, 0u,"),
    ("2D: tile amax from its first row only", "for (int i = 0; i < 16; ++i)\n        for (int j = 0; j < 16; ++j) {",
     "for (int i = 0; i < 1; ++i)\n        for (int j = 0; j < 16; ++j) {"),
    ("codes: nibbles swapped", "  if (k & 1)\n    row[k >> 1]", "  if (!(k & 1))\n    row[k >> 1]"),
    # dequantize and GEMM
    ("dequantize: multiplies by the tensor scale", "scales[i * (K / 16) + k / 16]) / s_enc;",
     "scales[i * (K / 16) + k / 16]) * s_enc;"),
    ("dequantize: scale of the wrong block", "scales[i * (K / 16) + k / 16]) / s_enc;",
     "scales[i * (K / 16) + k / 32]) / s_enc;"),
    ("gemm: signed sum for the tolerance", "    acc_abs += fabs(p);\n  }\n  *c = acc;",
     "    acc_abs += p;\n  }\n  *c = acc;"),
    ("gemm: last product left out", "  for (int64_t k = 0; k < K; ++k) {\n    const double p = deq(",
     "  for (int64_t k = 0; k < K - 1; ++k) {\n    const double p = deq("),
    ("block amax: signed maximum", "        if (fabsf(blk[j]) > amax_b) amax_b = fabsf(blk[j]);",
     "        if (blk[j] > amax_b) amax_b = blk[j];"),
    ("tensor scale: overflow not clamped", "  if (isinf(s)) s = FLT_MAX;\n  return s;", "  return s;"),
    ("multiplier: overflow not clamped", "*inv = isinf(q) ? FLT_MAX : q;", "*inv = q;"),
    ("multiplier: zero-scale block passes x through", "    *inv = 0.0f;\n  } else {", "    *inv = 1.0f;\n  } else {"),
    ("tensor scale: amax written as S_enc", "  tensor_scale[0] = s_enc;\n  tensor_scale[1] = amax;\n\n  /* rowwise",
     "  tensor_scale[0] = s_enc;\n  tensor_scale[1] = s_enc;\n\n  /* rowwise"),
    ("2D: transposed draw index", "seed, 0u, (uint64_t)(r * cols + c));\n          put_code(codes + r",
     "seed, 0u, (uint64_t)(c * rows + r));\n          put_code(codes + r"),
    ("2D: transposed scale of the wrong tile", "scales_t[(tc * 16 + j) * (rows / 16) + tr] = byte;",
     "scales_t[(tc * 16 + j) * (rows / 16) + tc % (rows / 16)] = byte;"),
    ("dequantize: nibbles swapped",
     "(k & 1) ? (byte >> 4) : (byte & 0x0F);\n  return orc_e2m1_value(code) * orc_e4m3_value",
     "(k & 1) ? (byte & 0x0F) : (byte >> 4);\n  return orc_e2m1_value(code) * orc_e4m3_value"),
    ("rht: difference the wrong way round", "v[i + h] = a - b;", "v[i + h] = b - a;"),
    ("draws: array form off by one", "orc_sr_bits(seed, stream, first + (uint64_t)i);",
     "orc_sr_bits(seed, stream, first + (uint64_t)i + 1);"),
    # MXFP4
    ("mx: scale exponent one too small", "int s = (e - 1) - 2;", "int s = (e - 1) - 1;"),
    ("mx: zero block takes byte 1", "if (amax == 0.0f) return -127;", "if (amax == 0.0f) return -126;"),
    ("mx: elements scaled one binade off", "ldexp((double)load_elem(x, dtype, r * cols + 32 * b + k), -s)",
     "ldexp((double)load_elem(x, dtype, r * cols + 32 * b + k), -s + 1)"),
    ("mx: block amax over half the block", "      for (int k = 0; k < 32; ++k) {\n        const float a = fabsf(",
     "      for (int k = 0; k < 16; ++k) {\n        const float a = fabsf("),
    ("mx: E8M0 bias 128", "return ldexp(1.0, (byte & 0xFF) - 127);", "return ldexp(1.0, (byte & 0xFF) - 128);"),
    ("mx: dequantize nibbles swapped", "(k & 1) ? (byte >> 4) : (byte & 0x0F);\n  return orc_e2m1_value(code) * orc_e8m0_value",
     "(k & 1) ? (byte & 0x0F) : (byte >> 4);\n  return orc_e2m1_value(code) * orc_e8m0_value"),
    ("rht: sign word from output word 1", "  return out[0] & 0xFFFFu;", "  return out[1] & 0xFFFFu;"),
    ("rht: one sign of the mask flipped", "      rht16(v, mask);", "      rht16(v, mask ^ 1u);"),
    ("philox: key halves swapped in the draws",
     "const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};",
     "const uint32_t key[2] = {(uint32_t)(seed >> 32), (uint32_t)seed};"),
    ("e4m3 decode: NaN at 0x7E", "if (e == 15 && m == 7) return NAN;", "if (e == 15 && m == 6) return NAN;"),
    ("dequantize: sign dropped", "return orc_e2m1_value(code) * orc_e4m3_value(scales[i * (K / 16) + k / 16]) / s_enc;",
     "return orc_e2m1_value(code & 7) * orc_e4m3_value(scales[i * (K / 16) + k / 16]) / s_enc;"),
    ("gemm: accumulated in float", "    const double p = deq(a_codes, a_scales, sa, K, i, k) * deq(b_codes, b_scales, sb, K, j, k);\n    acc += p;",
     "    const double p = deq(a_codes, a_scales, sa, K, i, k) * deq(b_codes, b_scales, sb, K, j, k);\n    acc = (float)(acc + p);"),
    ("input check: infinities accepted", "if (!isfinite(load_elem(x, dtype, i))) bad = 1;",
     "if (isnan(load_elem(x, dtype, i))) bad = 1;"),
    ("block scale: zero test on the wrong side", "  if (sb == 0.0f) {", "  if (sb < 0.0f) {"),
    ("quantize: transform ignored", "  if (rht) {\n    orc_rht(x, dtype, rows, cols, rht_seed, v);",
     "  if (0) {\n    orc_rht(x, dtype, rows, cols, rht_seed, v);"),
    ("mx: exponent not clamped below", "  if (s < -127) s = -127;\n", ""),
    ("mx: 16-element scale blocks in the GEMM", "orc_e8m0_value(scales[i * (K / 32) + k / 32])",
     "orc_e8m0_value(scales[i * (K / 32) + k / 16])"),
]


def test_mutants_are_well_formed():
    src = open(SRC).read()
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"{name}: the text to replace must occur exactly once"
        assert old != new


def _build(tmp, tag, text):
    d = os.path.join(tmp, tag)
    os.makedirs(d)
    src = os.path.join(d, "nvfp4_oracle.c")
    with open(src, "w") as f:
        f.write(text)
    shutil.copy(HDR, d)
    out = os.path.join(d, "liboracle.so")
    oracle.build(src=src, out=out)
    return out


def _run_pins(lib_path, threads):
    env = dict(os.environ, NVFP4_ORACLE_LIB=lib_path, OMP_NUM_THREADS=str(threads))
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *PIN_FILES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout[-2000:]


@pytest.mark.timeout(1800)
def test_every_mutant_fails_a_pin(tmp_path):
    base = open(SRC).read()
    jobs = [("original", base)] + [(f"m{k:02d}", base.replace(old, new)) for k, (_, old, new) in
                                   enumerate(MUTANTS)]
    cpus = os.cpu_count() or 4
    workers = max(1, min(8, cpus // 2))

    def one(job):
        tag, text = job
        return tag, _run_pins(_build(str(tmp_path), tag, text), 2)
    with ThreadPoolExecutor(workers) as pool:
        results = dict(pool.map(one, jobs))

    rc, out = results.pop("original")
    assert rc == 0, f"the unmutated oracle must pass its pins:\n{out}"
    survivors = []
    for k, (name, _, _) in enumerate(MUTANTS):
        rc, out = results[f"m{k:02d}"]
        # exit status 1 is "tests ran and some failed"; anything else is a
        # harness problem, not a caught mutant
        assert rc in (0, 1), f"{name}: child pytest exited with {rc}:\n{out}"
        if rc == 0:
            survivors.append(name)
    assert not survivors, f"mutants that no pin catches: {survivors}"
