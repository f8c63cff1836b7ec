"""Pin strength: plant a plausible mistake in a copy of the oracle source,
build it, and require at least one pin to catch it (CPU only)."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "csa2_oracle.c")

# (name, original text, mistaken text)
MUTANTS = [
    ("nibble_order", "return orc_e2m1((ch & 1) ? (b >> 4) : (b & 15u));",
     "return orc_e2m1((ch & 1) ? (b & 15u) : (b >> 4));"),
    ("e4m3_bias", "ldexp(1.0 + (double)m / 8.0, (int)e - 7)", "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    ("e8m0_bias", "(int)(byte & 0xFFu) - 127", "(int)(byte & 0xFFu) - 128"),
    ("e2m1_subnormal", "(e == 0) ? 0.5 * (double)m", "(e == 0) ? 1.0 * (double)m"),
    ("main_scale_group", "orc_e4m3(entry[256 + c / 16])", "orc_e4m3(entry[256 + c / 32])"),
    ("index_scale_group", "orc_e8m0(scales[c / 32])", "orc_e8m0(scales[c / 16 % 4])"),
    ("relu_after_weight", "acc += (double)w[q * 32 + h] * r;", "acc += fmax((double)w[q * 32 + h] * d, 0.0);"),
    ("dropped_head", "acc += (double)w[q * 32 + h] * r;", "if (h != 31) acc += (double)w[q * 32 + h] * r;"),
    ("reversed_key", "d += qv[h][c] * kv[c];", "d += qv[h][c] * kv[127 - c];"),
    ("pool_block_scale", "return 8 * (int64_t)blocks_q[p / 8] + p % 8;", "return (int64_t)blocks_q[p / 8] + p % 8;"),
    ("causal_off_by_one", "if (e < 0 || e >= limit) {\n        scores", "if (e < 0 || e >= limit - 1) {\n        scores"),
    ("tie_break_high_index", "return (x->e < y->e) ? -1 : (x->e > y->e) ? 1 : 0;",
     "return (x->e > y->e) ? -1 : (x->e < y->e) ? 1 : 0;"),
    ("ascending_scores", "return (x->s > y->s) ? -1 : 1;", "return (x->s < y->s) ? -1 : 1;"),
    ("no_softmax_scale", "lg[j] = scale * d;", "lg[j] = d;"),
    ("no_normalisation", "double p = exp(lg[j] - mx) / z;", "double p = exp(lg[j] - mx);"),
    ("swa_dropped", "for (int r = 0; r < n_swa; ++r) {", "for (int r = 0; r < n_swa - 1; ++r) {"),
    ("swa_row_stride", "swa + (size_t)((int64_t)qi * swa_q_stride + r) * 512", "swa + (size_t)((int64_t)qi * swa_q_stride) * 512"),
    ("wrong_head_query", "q_bf16[((size_t)qi * 64 + h) * 512 + c]", "q_bf16[((size_t)qi * 64 + (h ^ 1)) * 512 + c]"),
    ("lse_missing_max", "(float)(mx + log(z))", "(float)(log(z))"),
    ("quant_ties_to_odd", "(m & 1u) == 0 && (best_m & 1u) == 1", "(m & 1u) == 1 && (best_m & 1u) == 0"),
    ("quant_scale_over_4", "double d = fabs(amax - 6.0 * orc_e4m3(c));", "double d = fabs(amax - 4.0 * orc_e4m3(c));"),
    ("quant_no_e4m3_saturation", "if (amax > 6.0 * 448.0) amax = 6.0 * 448.0;", ""),
    ("quant_mx_floor_at_powers", "6.0 * ldexp(1.0, e) < amax", "6.0 * ldexp(1.0, e) <= amax"),
    ("quant_mx_scale_over_4", "6.0 * ldexp(1.0, e) < amax", "4.0 * ldexp(1.0, e) < amax"),
    ("quant_sign_of_zero", "signbit(x) ? 8u : 0u", "(x < 0.0f) ? 8u : 0u"),
    ("quant_nibble_order", "codes[ch >> 1] |= (uint8_t)(code << ((ch & 1) ? 4 : 0));",
     "codes[ch >> 1] |= (uint8_t)(code << ((ch & 1) ? 0 : 4));"),
    ("quant_zero_scale_codes", "if (s == 0.0) continue;", ""),
    ("quant_amax_one_channel", "double a = abs_or_zero(xi[16 * g + c]);", "double a = abs_or_zero(xi[16 * g]);"),
    ("swa_fp8_scale_block", "orc_e8m0(row[512 + c / 32])", "orc_e8m0(row[512 + c / 16 % 16])"),
    ("swa_fp8_row_stride", "* 528, kv + (size_t)nj * 512);", "* 512, kv + (size_t)nj * 512);"),
    ("rope_sign", "o[449 + 2 * i] = b * cs - a * sn;", "o[449 + 2 * i] = b * cs + a * sn;"),
    ("rope_offset", "double a = o[448 + 2 * i], b = o[449 + 2 * i];", "double a = o[446 + 2 * i], b = o[447 + 2 * i];"),
    ("rope_cos_sin_swapped", "double cs = rope_cs[((size_t)qi * 32 + i) * 2], sn = rope_cs[((size_t)qi * 32 + i) * 2 + 1];",
     "double sn = rope_cs[((size_t)qi * 32 + i) * 2], cs = rope_cs[((size_t)qi * 32 + i) * 2 + 1];"),
    ("pool_block_of_4", "for (int64_t e = 8 * b; e < 8 * b + 8 && e < lim; ++e) {",
     "for (int64_t e = 8 * b; e < 8 * b + 4 && e < lim; ++e) {"),
    ("pool_min_not_max", "if (e == 8 * b || score_better(x, best)) best = x;",
     "if (e == 8 * b || score_better(best, x)) best = x;"),
    ("pool_ignores_limit", "for (int64_t e = 8 * b; e < 8 * b + 8 && e < lim; ++e) {",
     "for (int64_t e = 8 * b; e < 8 * b + 8 && e < n_entries; ++e) {"),
    ("pool_nan_ranks_high", "  if (isnan(x)) return 0;\n  if (isnan(y)) return 1;", "  if (isnan(x)) return 1;\n  if (isnan(y)) return 0;"),
    ("gate_sign", "double pa = 1.0 / (1.0 + exp(gb - ga)), pb", "double pa = 1.0 / (1.0 + exp(ga - gb)), pb"),
    ("gate_one_channel", "int gc = gate_width == 1 ? 0 : c;", "int gc = 0;"),
    ("pooled_same_token", "const float* xb = xa + 512;", "const float* xb = xa;"),
    ("gather_wrong_query", "main_cache + (size_t)((int64_t)q * cache_q_stride + e) * 288, 288);",
     "main_cache + (size_t)((int64_t)0 * cache_q_stride + e) * 288, 288);"),
    ("gather_dense_id", "dense_idx[(size_t)q * k + j] = ok ? j : -1;", "dense_idx[(size_t)q * k + j] = ok ? (int)e : -1;"),
    ("bf16_through_f32", "  uint64_t u;\n  memcpy(&u, &v, 8);", "  uint64_t u;\n  v = (double)(float)v;\n  memcpy(&u, &v, 8);"),
    ("bf16_ties_away", "if (rem > half || (rem == half && (keep & 1))) ++keep;", "if (rem >= half) ++keep;"),
    ("bf16_truncate", "if (rem > half || (rem == half && (keep & 1))) ++keep;", ""),
    ("quant_mx_zero_block", "if (amax > 0.0) {\n        e = -127;", "if (amax >= 0.0) {\n        e = -127;"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / f"mut_{name}.c"
    mut.write_text(src.replace(orig, bad))
    so = str(tmp_path / f"libmut_{name}.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", str(mut), "-o", so, "-lm"],
                   check=True)
    L = oracle.load_variant(so)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(L)
        except AssertionError:
            caught.append(check.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
