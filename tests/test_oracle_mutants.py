"""Each mutant is the oracle's C source with one plausible mistake planted
(a wrong index, a dropped term, a wrong constant or rounding rule).  The pins
must reject every mutant; this shows they are strong enough to trust the
oracle.  The mistakes are planted only in temporary copies, on the CPU."""

import os

import pytest

import oracle
import oracle_pins as pins

MUTANTS = {
    "rank_round_robin": ("is_token_in_rank[(int64_t)t * R + e / epr] = 1;",
                         "is_token_in_rank[(int64_t)t * R + e % R] = 1;"),
    "slot_descending": ("send_slot[i] = rank_offset[r] + c;",
                        "send_slot[i] = rank_offset[r + 1] - 1 - c;"),
    "drop_counted_as_expert0": ("if (e == -1) continue;\n            if (e < -1",
                                "if (e == -1) e = 0;\n            if (e < -1"),
    "expert_scan_off": ("expert_offset[e + 1] = expert_offset[e] + num_tokens_per_expert[e];",
                        "expert_offset[e + 1] = expert_offset[e] + num_tokens_per_expert[e] - (e == 0);"),
    "e4m3_ties_away": ("double m = nearbyint(ldexp(a, 3 - E));",
                       "double m = round(ldexp(a, 3 - E));"),
    "e4m3_sub_ties_away": ("double m = nearbyint(ldexp(a, 9));",
                           "double m = round(ldexp(a, 9));"),
    "e4m3_bias8": ("int code = ((E + 7) << 3) | ((int)m - 8);",
                   "int code = ((E + 8) << 3) | ((int)m - 8);"),
    "e4m3_overflow_nan": ("if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
                          "if (a >= 448.0) return (uint8_t)(sign | 0x7F);"),
    "e4m3_sign_dropped": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;",
                          "uint8_t sign = 0x00;"),
    "quant_max_not_abs": ("float v = fabsf(bf16_to_float(xrow[b * 128 + i]));",
                          "float v = bf16_to_float(xrow[b * 128 + i]);"),
    "quant_scale_inverted": ("float s = a / 448.0f;", "float s = 448.0f / a;"),
    "quant_divide_by_scale": ("float prod = xv * inv;", "float prod = xv / (a / 448.0f);"),
    "quant_nan_in_amax": ("if (v > amax) amax = v;", "if (!(v <= amax)) amax = v;"),
    "quant_nan_sign_dropped": ("(uint8_t)((signbit(xv) ? 0x80 : 0x00) | 0x7F);", "(uint8_t)0x7F;"),
    "row_pitch_unpadded": ("return (payload + 127) / 128 * 128;", "return payload;"),
    "row_pad_short": ("i < pitch; i++) out_row[i] = 0;", "i < pitch - 4; i++) out_row[i] = 0;"),
    "quant_block_64": ("float amax = 0.0f;\n        for (int i = 0; i < 128; i++) {",
                       "float amax = 0.0f;\n        for (int i = 0; i < 64; i++) {"),
    "meta_global_expert": ("slot_local_idx[(int64_t)s * k + j] = local ? e - r * epr : -1;",
                           "slot_local_idx[(int64_t)s * k + j] = local ? e : -1;"),
    "meta_weight_unmasked": ("slot_local_w[(int64_t)s * k + j] = local ? topk_w[(int64_t)t * k + j] : 0.0f;",
                             "slot_local_w[(int64_t)s * k + j] = topk_w[(int64_t)t * k + j];"),
    "desc_abs_dst_offset": ("d.dst_offset = (uint64_t)(8LL * m) * (uint64_t)row_bytes;",
                            "d.dst_offset = (uint64_t)(rank_offset[r] + 8LL * m) * (uint64_t)row_bytes;"),
    "desc_atomic_msgs": ("a.size_or_value = (uint32_t)cnt;",
                         "a.size_or_value = (uint32_t)((cnt + 7) / 8);"),
    "desc_batch_7": ("if (rows > 8) rows = 8;", "if (rows > 7) rows = 7;"),
    "combine_drop_counted": ("if (e < 0) continue;\n            W[e / epr]",
                             "if (e < -1) continue;\n            W[e / epr]"),
    "combine_rank_map": ("W[e / epr] += (double)topk_w", "W[e % R] += (double)topk_w"),
    "combine_unweighted": ("o[h] += W[r] * (double)bf16_to_float(yrow[h]);",
                           "o[h] += (double)bf16_to_float(yrow[h]);"),
    "ll_slot_descending": ("expert_slot[i] = expert_offset[e] + run[e]++;",
                           "expert_slot[i] = expert_offset[e + 1] - 1 - run[e]++;"),
    "ll_drop_counted": ("if (e == -1) continue;\n        if (e < -1 || e >= E) { status = ORC_ERR_BAD_EXPERT; continue; }",
                        "if (e == -1) e = 0;\n        if (e < -1 || e >= E) { status = ORC_ERR_BAD_EXPERT; continue; }"),
    "ll_dst_absolute": ("d.dst_offset = (uint64_t)(expert_offset[e] - base + 8LL * m) * (uint64_t)row_bytes;",
                        "d.dst_offset = (uint64_t)(expert_offset[e] + 8LL * m) * (uint64_t)row_bytes;"),
    "ll_atomic_global_expert": ("a.dst_offset = (uint64_t)(4 * le);", "a.dst_offset = (uint64_t)(4 * e);"),
    "ll_batch_7": ("int32_t rows = cnt - 8 * m < 8 ? cnt - 8 * m : 8;",
                   "int32_t rows = cnt - 8 * m < 7 ? cnt - 8 * m : 7;"),
    "ll_meta_first_gate": ("slot_w[s] = topk_w[(int64_t)t * k + j];", "slot_w[s] = topk_w[(int64_t)t * k];"),
    "ll_combine_unweighted": ("o[h] += w * (double)bf16_to_float(yrow[h]);",
                              "o[h] += (double)bf16_to_float(yrow[h]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.compile_source(str(path), str(tmp_path / "libmutant.so"))
    O = oracle.Oracle(so)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
            break
    assert failed, f"no pin rejects mutant {name}"
