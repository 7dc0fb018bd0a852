"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (CPU only).  A mutant that survived would mean the pins do not
pin that part of the oracle."""
import os

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kvq_oracle.c")

# (id, original text, planted mistake, occurrence to replace, pins that must catch it)
MUTANTS = [
    ("int8_step_128", "float s = fmaxf(a, 1e-8f) / 127.0f;", "float s = fmaxf(a, 1e-8f) / 128.0f;", 0,
     [pins.pin_int8_pth]),
    ("ties_away", "return (lo % 2 == 0) ? lo : hi;", "return hi;", 0,
     [pins.pin_e4m3_encode, pins.pin_e2m1_encode]),
    ("nvfp4_block_max_to_4", "kvqo_e4m3_encode((a / 6.0f) / st)", "kvqo_e4m3_encode((a / 4.0f) / st)", 0,
     [pins.pin_nvfp4]),
    ("wht_sign", "y[j + h] = a - b;", "y[j + h] = b - a;", 0, [pins.pin_kvarn_rotation]),
    ("kvarn_no_channel_division", "for (int t = 0; t < N; t++) Y[t * N + j] = Y[t * N + j] * inv;",
     "(void)0;", 0, [pins.pin_kvarn_tile]),
    ("kvarn_dev_scale", "float sd = sqrtf(sum_tree(sq, 128) * 0.0078125f);",
     "float sd = sqrtf(sum_tree(sq, 128) * 0.015625f);", 0, [pins.pin_kvarn_tile]),
    ("nvfp4_v_nibble_index", "put_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2, cv[d]);",
     "put_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 2, d % 2, cv[d]);", 0, [pins.pin_layout_bijective]),
    ("gqa_modulo", "int kvh = h / G;", "int kvh = h % H;", 0, [pins.pin_attention]),
    ("softmax_scale_dropped", "lg[t] = acc * scale;", "lg[t] = acc;", 0, [pins.pin_attention]),
    ("e4m3_bias", "v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);", 0,
     [pins.pin_e4m3_decode]),
    ("kvarn_k_levels_16", "const float levels = side == 0 ? 15.0f : 3.0f;",
     "const float levels = side == 0 ? 16.0f : 3.0f;", 0, [pins.pin_kvarn_tile]),
    ("fp8_max_fnuz", "float s = fmaxf(a, 1e-8f) / 448.0f;", "float s = fmaxf(a, 1e-8f) / 240.0f;", 0,
     [pins.pin_fp8_pth]),
    ("four_over_six_inverted", "if (e4 < e6) {", "if (e4 > e6) {", 0, [pins.pin_nvfp4]),
    ("half_subnormal_exp", "v = ldexpf((float)m, -24);", "v = ldexpf((float)m, -25);", 0,
     [pins.pin_half_widening]),
    ("kvarn_alpha_without_c", "meta[i] = c[i] * s_q[i];", "meta[i] = s_q[i];", 0, [pins.pin_kvarn_tile]),
    ("v8_row_major_store", "vc[v8_off(D, t, d)] = cv[d];", "vc[(int64_t)t * D + d] = cv[d];", 0,
     [pins.pin_glossary_bytes]),
    ("k8_offset_swizzle", "return 16LL * D * u + 64 * B * h + 16 * B * g + B * s + e;",
     "return 16LL * D * u + 64 * B * h + 16 * B * s + B * g + e;", 0, [pins.pin_layout_bijective]),
    ("int4_k_nibble_order", "put_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2, ck[d]);",
     "put_nibble(kc + (int64_t)t * D / 2 + d / 2, 1 - d % 2, ck[d]);", 0, [pins.pin_int4_pth]),
    ("int4_step_8", "float s = fmaxf(a, 1e-8f) / 7.0f;", "float s = fmaxf(a, 1e-8f) / 8.0f;", 0,
     [pins.pin_int4_pth]),
    ("int4_unsigned_decode", "k[d] = (double)((a ^ 8) - 8) * (double)tmp[0];", "k[d] = (double)a * (double)tmp[0];", 0,
     [pins.pin_int4_pth]),
    ("mxfp4_emax_1", "int k = (ex - 1) - 2;", "int k = (ex - 1) - 1;", 0, [pins.pin_mxfp4]),
    ("mxfp4_ceil_exponent", "int k = (ex - 1) - 2;", "int k = ex - 2;", 0, [pins.pin_mxfp4]),
    ("mxfp4_unbiased_byte", "bscales[b] = (uint8_t)(k + 127);", "bscales[b] = (uint8_t)(k + 128);", 0,
     [pins.pin_mxfp4]),
    ("mxfp4_v_scale_token_major", "vs[(int64_t)b * P + t] = bv[b];", "vs[(int64_t)t * (D / BL) + b] = bv[b];", 0,
     [pins.pin_mxfp4, pins.pin_layout_bijective]),
    ("mxfp4_decode_scale_block_16", "(int)ks[(int64_t)t * (D / 32) + d / 32] - 127",
     "(int)ks[(int64_t)t * (D / 32) + d / 16 % (D / 32)] - 127", 0, [pins.pin_mxfp4]),
    ("kvarn_second_tile_over_first", "uint8_t* ch = chunk_at(L, cache, page, h) + (s0 % P) / 128 * KVARN_TILE_BYTES;",
     "uint8_t* ch = chunk_at(L, cache, page, h);", 0, [pins.pin_kvarn_pages, pins.pin_layout_bijective]),
    ("kvarn_read_first_tile", "ch += (int64_t)(t / 128) * KVARN_TILE_BYTES;", "(void)0;", 0, [pins.pin_kvarn_pages]),
    ("int8_floor_after_divide", "float s = fmaxf(a, 1e-8f) / 127.0f;", "float s = fmaxf(a / 127.0f, 1e-8f);", 0,
     [pins.pin_int_rule_order]),
    ("int8_reciprocal_product", "float y = x[d] / s;", "float y = x[d] * (1.0f / s);", 0,
     [pins.pin_int_rule_order]),
    ("int4_floor_after_divide", "float s = fmaxf(a, 1e-8f) / 7.0f;", "float s = fmaxf(a / 7.0f, 1e-8f);", 0,
     [pins.pin_int_rule_order]),
    ("int4_reciprocal_product", "float y = x[d] / s;", "float y = x[d] * (1.0f / s);", 1,
     [pins.pin_int_rule_order]),
    ("fp8_pth_reciprocal_product", "codes[d] = kvqo_e4m3_encode(x[d] / s);",
     "codes[d] = kvqo_e4m3_encode(x[d] * (1.0f / s));", 0, [pins.pin_fp8_pth]),
    ("kvarn_three_sweeps", "#define KVARN_ITERS 4", "#define KVARN_ITERS 3", 0, [pins.pin_kvarn_sweeps]),
    ("kvarn_eight_sweeps", "#define KVARN_ITERS 4", "#define KVARN_ITERS 8", 0, [pins.pin_kvarn_sweeps]),
    ("nvfp4_scale_divisor_product", "kvqo_e4m3_encode((a / 6.0f) / st)", "kvqo_e4m3_encode(a / (6.0f * st))", 0,
     [pins.pin_nvfp4_scale_order]),
    ("chunk_head_major", "return (uint8_t*)cache + (page * L->num_kv_heads + h) * kvqo_chunk_bytes(L);",
     "return (uint8_t*)cache + ((int64_t)h * L->num_pages + page) * kvqo_chunk_bytes(L);", 0,
     [pins.pin_layout_bijective]),
]


@pytest.mark.parametrize("mid,old,new,occ,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, old, new, occ, catchers):
    src = open(SRC).read()
    assert old in src, f"mutation site for {mid} not found"
    parts = src.split(old)
    assert len(parts) > occ + 1
    mutated = old.join(parts[:occ + 1]) + new + old.join(parts[occ + 1:])
    mpath = tmp_path / "mutant.c"
    mpath.write_text(mutated)
    so = oracle.build(force=True, src=str(mpath), out=str(tmp_path / "libmutant.so"))
    O = oracle.Oracle(so)
    caught = []
    for pin in catchers:
        try:
            pin(O)
        except (AssertionError, ValueError) as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {mid} survived {[p.__name__ for p in catchers]}"
