"""Plants plausible mistakes in copies of the CPU oracle and checks that the pins catch
each one (a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
rounding rule).  Runs entirely on the CPU; each mutant is built with gcc in a temporary
directory and exercised in a child process, so a mutant that crashes is caught too.
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "cf_oracle.c")
PINS = os.path.join(ROOT, "tests", "pins.py")

# (name, text in cf_oracle.c, replacement)
MUTANTS = [
    ("ef_error_sign",
     "d[i];\n            err[base + i] = act(dtype, a, base + i) - ahat[base + i];",
     "d[i];\n            err[base + i] = ahat[base + i] - act(dtype, a, base + i);"),
    ("update_sign",
     "ahat[base + i] = ahat[base + i] + d[i];\n            err[base + i] = act",
     "ahat[base + i] = ahat[base + i] - d[i];\n            err[base + i] = act"),
    ("residual_drops_ahat",
     "for (int i = 0; i < CFO_GROUP; ++i) r[i] = act(dtype, a, base + i) - ahat[base + i];",
     "for (int i = 0; i < CFO_GROUP; ++i) r[i] = act(dtype, a, base + i);"),
    ("q1_mean_divisor", "return ldexpf((float)q, low - 156);", "return ldexpf((float)q, low - 155);"),
    ("q1_implicit_bit", "(uint64_t)(mant | 0x800000u)", "(uint64_t)mant"),
    ("q1_exponent_offset", "int shift = expo ? (int)expo - 1 : 0;", "int shift = expo ? (int)expo : 0;"),
    ("q1_carry_dropped", "carry = t >> 32;\n            add >>= 32;", "carry = 0;\n            add >>= 32;"),
    ("q1_signed_sum", "float x = fabsf(r[i]);\n        uint32_t u;", "float x = r[i] < 0.0f ? 0.0f : r[i];\n        uint32_t u;"),
    ("q1_ties_away", "if (half && (rest || (q & 1u))) q += 1;", "if (half) q += 1;"),
    ("q1_sticky_ignored", "if (half && (rest || (q & 1u))) q += 1;", "if (half && (q & 1u)) q += 1;"),
    ("q1_truncates", "if (half && (rest || (q & 1u))) q += 1;", "(void)half; (void)rest;"),
    ("q1_subnormal_last_bit", "int low = top - 23 > 7 ? top - 23 : 7;", "int low = top - 23 > 6 ? top - 23 : 6;"),
    ("q1_code_sign", "c = r[i] < 0.0f ? 1u : 0u;", "c = r[i] > 0.0f ? 1u : 0u;"),
    ("q1_bit_order", "gcodes[i >> 3] |= (uint8_t)(c << (i & 7));",
     "gcodes[i >> 3] |= (uint8_t)(c << (7 - (i & 7)));"),
    ("q1_decode_sign", "if (bits == 1) return (c & 1u) ? -s : s;",
     "if (bits == 1) return (c & 1u) ? s : -s;"),
    ("q2_scale_reciprocal", "return M / 1.5f;", "return M * (1.0f / 1.5f);"),
    ("q2_scale_divisor", "return M / 1.5f;", "return M / 2.0f;"),
    ("q2_tie_rule", "unsigned mag = fabsf(r[i]) > s ? 1u : 0u;",
     "unsigned mag = fabsf(r[i]) >= s ? 1u : 0u;"),
    ("q2_outer_level", "float lvl = (c & 2u) ? 1.5f * s : 0.5f * s;",
     "float lvl = (c & 2u) ? 2.0f * s : 0.5f * s;"),
    ("q2_code_fields", "c = sign | (mag << 1);", "c = mag | (sign << 1);"),
    ("q2_pack_shift", "gcodes[i >> 2] |= (uint8_t)(c << (2 * (i & 3)));",
     "gcodes[i >> 2] |= (uint8_t)(c << (i & 3));"),
    ("decode_scale_index",
     "ahat[k] = ahat[k] + dequant(bits, code_at(bits, gc, i), scales[g]);",
     "ahat[k] = ahat[k] + dequant(bits, code_at(bits, gc, i), scales[g > 0 ? g - 1 : 0]);"),
    ("init_error_not_cleared", "if (err) err[i] = 0.0f;", "if (err) err[i] = ahat[i] * 0.5f;"),
    ("int4_divisor", "scales[j] = M / 7.0f;", "scales[j] = M / 8.0f;"),
    ("int4_rounding", "float q = rintf(x[i * k + j] / s);", "float q = roundf(x[i * k + j] / s);"),
    ("int4_nibble_order", "packed[(i * k + j) / 2] |= (uint8_t)((j & 1) ? nib << 4 : nib);",
     "packed[(i * k + j) / 2] |= (uint8_t)((j & 1) ? nib : nib << 4);"),
    ("int4_sign_extend", "int c = nib >= 8 ? nib - 16 : nib;", "int c = nib;"),
    ("householder_beta", "beta[j] = 2.0 / vv;", "beta[j] = 1.0 / vv;"),
    ("householder_guard_high", "alive[j] = fabs(rj) > 1e-5 * fro;", "alive[j] = fabs(rj) > 1e-2 * fro;"),
    ("householder_guard_low", "alive[j] = fabs(rj) > 1e-5 * fro;", "alive[j] = fabs(rj) > 1e-12 * fro;"),
    ("householder_reverse_order", "for (int j = steps - 1; j >= 0; --j) {",
     "for (int j = 0; j < steps; ++j) {"),
    ("backproject_column", "for (int j = 0; j < k; ++j) Q[l * k + j] += ril * P[i * k + j];",
     "for (int j = 0; j < k; ++j) Q[l * k + j] += ril * P[i * k + (k - 1 - j)];"),
    ("project_transposed_q", "for (int64_t l = 0; l < n; ++l) s += (double)r[i * n + l] * Q[l * k + j];",
     "for (int64_t l = 0; l < n; ++l) s += (double)r[i * n + l] * Q[(l % k) * k + (j % k)];"),
    ("lowrank_update_sign", "ahat[i * n + l] = ahat[i * n + l] + (float)s;\n            err[",
     "ahat[i * n + l] = ahat[i * n + l] - (float)s;\n            err["),
    ("lowrank_single_iteration", "for (int it = 0; it < iters; ++it) {",
     "for (int it = 0; it < 1; ++it) {"),
    ("lowrank_receiver_dequant_v",
     "cfo_int4_dequantize((const uint8_t*)v, v_scales, n, k, Vh);\n    } else if (factor_bits == 16) {\n        for (int64_t i = 0; i < m * k; ++i) Uh[i] = bf16_widen",
     "cfo_int4_dequantize((const uint8_t*)v, u_scales, n, k, Vh);\n    } else if (factor_bits == 16) {\n        for (int64_t i = 0; i < m * k; ++i) Uh[i] = bf16_widen"),
    ("explicit_ef_error_sign", "err[base + i] = r[i] - d[i];", "err[base + i] = d[i] - r[i];"),
    ("bf16_truncates", "return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);",
     "return (uint16_t)(u >> 16);"),
    ("noef_residual_uses_mirror",
     "r[i] = act(dtype, a, base + i) - act(dtype, a_prev, base + i);",
     "r[i] = act(dtype, a, base + i) - ahat[base + i];"),
    ("noef_mirror_not_updated",
     "for (int i = 0; i < CFO_GROUP; ++i) ahat[base + i] = ahat[base + i] + d[i];",
     "for (int i = 0; i < CFO_GROUP; ++i) ahat[base + i] = ahat[base + i];"),
    ("naive_input_scaled", "for (int i = 0; i < CFO_GROUP; ++i) r[i] = act(dtype, a, base + i);",
     "for (int i = 0; i < CFO_GROUP; ++i) r[i] = 0.5f * act(dtype, a, base + i);"),
    ("topk_ties_to_higher_index", "return i < j ? -1 : (i > j);\n}\n\nstatic int by_index",
     "return i > j ? -1 : (i < j);\n}\n\nstatic int by_index"),
    ("topk_keeps_smallest", "if (ki != kj) return ki > kj ? -1 : 1;",
     "if (ki != kj) return ki < kj ? -1 : 1;"),
    ("topk_signed_key", "float m = fabsf(r);", "float m = r;"),
    ("topk_output_unsorted", "qsort(order, (size_t)k, sizeof(int), by_index);", "(void)by_index;"),
    ("topk_value_truncated", "uint16_t h = bf16_rne(r[i]);",
     "uint16_t h = (uint16_t)(mag_key(r[i]) >> 16) | (r[i] < 0.0f ? 0x8000u : 0u);"),
    ("topk_one_slot_short", "for (int j = 0; j < k; ++j) {\n            int i = order[j];",
     "for (int j = 0; j < k - 1; ++j) {\n            int i = order[j];"),
    ("topk_sender_unrounded", "ahat[base + i] = ahat[base + i] + bf16_widen(h);",
     "ahat[base + i] = ahat[base + i] + r[i];"),
    ("topk_decode_slot_as_index", "int64_t e = g * CFO_GROUP + (idx[g * k + j] & 127);",
     "int64_t e = g * CFO_GROUP + j;"),
    ("topk_decode_group_stride", "int64_t e = g * CFO_GROUP + (idx[g * k + j] & 127);",
     "int64_t e = g * k + (idx[g * k + j] & 127);"),
]


@pytest.fixture(scope="module")
def workdir():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp(prefix="cfo_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_mutation_list_is_current():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutant {name}: pattern found {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1
    c_path = os.path.join(workdir, f"{name}.c")
    so_path = os.path.join(workdir, f"lib_{name}.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", so_path, c_path,
                    "-lm"], check=True, capture_output=True)
    p = subprocess.run([sys.executable, PINS, so_path], capture_output=True, text=True, timeout=300)
    if p.returncode != 0:
        return  # the mutant crashed the pin run: caught
    res = json.loads(p.stdout.strip().splitlines()[-1])
    failed = [k for k, v in res.items() if v is not None]
    assert failed, f"mutant {name} passed every pin"
