"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a one-spot textual edit of ``oracle/ep_oracle.c`` (a dropped
term, a wrong index or sign, a transposed operand, an off-by-one), compiled
with gcc into a temporary library and run through the pins in a child
process, so a mutant that crashes cannot take the test run down with it
(a crash on a signal counts as caught).  Runs on the CPU only.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ep_oracle.c")

MUTANTS = {
    "rank_of_expert_modulo": ("row[e / experts_per_rank] = 1;", "row[e % R] = 1;"),
    "expert_count_dropped": ("num_tokens_per_expert[e] += 1;", ";"),
    "node_skips_first_rank": ("for (int32_t r = n * 8; r < R && r < (n + 1) * 8; ++r) any |= row[r];",
                              "for (int32_t r = n * 8 + 1; r < R && r < (n + 1) * 8; ++r) any |= row[r];"),
    "node_size_four": ("for (int32_t r = n * 8; r < R && r < (n + 1) * 8; ++r) any |= row[r];",
                       "for (int32_t r = n * 4; r < R && r < (n + 1) * 4; ++r) any |= row[r];"),
    "channel_len_floor": ("int64_t tc = (T + C - 1) / C;", "int64_t tc = T / C;"),
    "gbl_transposed": ("gbl_channel_prefix_matrix[(int64_t)r * C + c] = running;",
                       "gbl_channel_prefix_matrix[(int64_t)c * R + r] = running;"),
    "rdma_counts_ranks_not_tokens": ("any |= is_token_in_rank[t * R + r] != 0;",
                                     "any += is_token_in_rank[t * R + r] != 0;"),
    "recv_prefix_exclusive": ("sum += num_tokens_per_rank[r];\n        recv_gbl_rank_prefix_sum[r] = sum;",
                              "recv_gbl_rank_prefix_sum[r] = sum;\n        sum += num_tokens_per_rank[r];"),
    "alignment_floor": ("(n + expert_alignment - 1) / expert_alignment * expert_alignment",
                        "n / expert_alignment * expert_alignment"),
    "slab_base_off_by_one": ("r > 0 ? recv_gbl_rank_prefix_sum[r - 1] : 0;",
                             "r > 1 ? recv_gbl_rank_prefix_sum[r - 2] : 0;"),
    "local_id_unscaled": ("on_r ? e - (int64_t)r * experts_per_rank : -1", "on_r ? e - (int64_t)r : -1"),
    "weights_unmasked": ("recv_topk_weights[row * K + j] = on_r ? topk_weights[t * K + j] : 0.0f;",
                         "recv_topk_weights[row * K + j] = topk_weights[t * K + j];"),
    "src_idx_is_row": ("recv_src_info[row * 2 + 1] = (int32_t)t;", "recv_src_info[row * 2 + 1] = (int32_t)row;"),
    "src_rank_dropped": ("recv_src_info[row * 2 + 0] = my_rank;", "recv_src_info[row * 2 + 0] = 0;"),
    "tokens_descending_in_channel": (
        "for (int64_t t = orc_channel_begin(T, C, c); t < orc_channel_end(T, C, c); ++t) {\n"
        "                if (!is_token_in_rank[t * R + r]) continue;",
        "for (int64_t t = orc_channel_end(T, C, c) - 1; t >= orc_channel_begin(T, C, c); --t) {\n"
        "                if (!is_token_in_rank[t * R + r]) continue;"),
    "W_keeps_last_term": ("W = W + recv_topk_weights[(int64_t)s * K + j];", "W = recv_topk_weights[(int64_t)s * K + j];"),
    "combine_reads_rank_row": ("const uint16_t *yrow = y + (int64_t)s * H;",
                               "const uint16_t *yrow = y + (int64_t)(s > 0 ? s - 1 : s) * H;"),
    "combine_fma_operands_swapped": ("fmaf(W, orc_bf16_to_f32(yrow[i]), acc_scratch[i])",
                                     "fmaf(acc_scratch[i], orc_bf16_to_f32(yrow[i]), W)"),
    "combined_weights_last_only": (
        "combined_topk_weights[t * K + j] = combined_topk_weights[t * K + j] + recv_topk_weights[(int64_t)s * K + j];",
        "combined_topk_weights[t * K + j] = recv_topk_weights[(int64_t)s * K + j];"),
    "rounding_ties_away": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
                           "if (dropped >= 0x8000u) kept += 1u;"),
    "rounding_truncates": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;", ";"),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "fp8_scales_not_copied": ("recv_x_scales[row * num_scales + i] = x_scales[t * num_scales + i];", ";"),
    "cached_wrong_source_row": ("memcpy(recv_x + s * row_bytes, x + t * row_bytes, (size_t)row_bytes);",
                                "memcpy(recv_x + s * row_bytes, x + (t > 0 ? t - 1 : t) * row_bytes, (size_t)row_bytes);"),
    "cached_bad_slot_not_flagged": ("                status |= ORC_BAD_SEND_SLOT;\n                continue;\n            }\n            memcpy(recv_x",
                                    "                continue;\n            }\n            memcpy(recv_x"),
    "last_column_unchecked": ("if (row != slab_begin + gbl_channel_prefix_matrix[(int64_t)r * C + C - 1]) status |= ORC_COUNT_MISMATCH;",
                              ";"),
    "segment_start_unchecked": ("if (row != seg_begin) status |= ORC_COUNT_MISMATCH;", ";"),
    "combine_f64_keeps_last_rank": ("o[i] += W * (double)orc_bf16_to_f32(y[(int64_t)s * H + i]);",
                                    "o[i] = W * (double)orc_bf16_to_f32(y[(int64_t)s * H + i]);"),
    "combine_f64_W_keeps_last_term": ("W += (double)recv_topk_weights[(int64_t)s * K + j];",
                                      "W = (double)recv_topk_weights[(int64_t)s * K + j];"),
    "group_slot_major_order": ("for (int64_t row = lo; row < hi; ++row) {\n                for (int32_t j = 0; j < K; ++j) {",
                               "for (int32_t j = 0; j < K; ++j) {\n                for (int64_t row = lo; row < hi; ++row) {"),
    "group_offsets_unaligned": ("offset += size;", "offset += used;"),
    "group_local_id_as_global": ("if (recv_topk_idx[row * K + j] != le) continue;",
                                 "if (recv_topk_idx[row * K + j] != e) continue;"),
    "group_padding_row_not_marked": ("grouped_row[pos] = -1;", "grouped_row[pos] = 0;"),
    "group_weight_of_slot0": ("grouped_weights[pos] = recv_topk_weights[row * K + j];",
                              "grouped_weights[pos] = recv_topk_weights[row * K];"),
    "group_segment_bound_ignored": ("if (used >= size || pos >= grouped_capacity) {",
                                    "if (pos >= grouped_capacity) {"),
    "e4m3_bias_eight": ("code = (uint8_t)(((E + 7) << 3) | ((int)q - 8));",
                        "code = (uint8_t)(((E + 8) << 3) | ((int)q - 8));"),
    "e4m3_ties_away": ("double q = rint(ldexp(mag, 3 - E));", "double q = floor(ldexp(mag, 3 - E) + 0.5);"),
    "e4m3_truncates": ("double q = rint(ldexp(mag, 3 - E));", "double q = floor(ldexp(mag, 3 - E));"),
    "e4m3_subnormal_step": ("code = (uint8_t)rint(ldexp(mag, 9));", "code = (uint8_t)rint(ldexp(mag, 10));"),
    "e4m3_subnormal_ties_away": ("code = (uint8_t)rint(ldexp(mag, 9));",
                                 "code = (uint8_t)floor(ldexp(mag, 9) + 0.5);"),
    "e4m3_normal_threshold": ("if (mag >= ldexp(1.0, -6)) {", "if (mag >= ldexp(1.0, -7)) {"),
    "e4m3_sign_dropped": ("return signbit(v) ? (uint8_t)(code | 0x80) : code;", "return code;"),
    "e4m3_decode_no_subnormals": (
        "double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);",
        "double mag = ldexp(1.0 + man / 8.0, ex - 7);"),
    "e4m3_decode_bias": (
        "double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);",
        "double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 8);"),
    "e4m3_decode_nan_pattern": ("if (ex == 15 && man == 7) return NAN;", "if (ex == 15 && man == 6) return NAN;"),
    "quant_scale_divisor": ("scales[t * num_scales + q] = a / 448.0f;", "scales[t * num_scales + q] = a / 240.0f;"),
    "quant_inverse_numerator": ("const float inv = 448.0f / a;", "const float inv = 240.0f / a;"),
    "quant_amax_signed": ("const float m = fabsf(orc_bf16_to_f32(xg[i]));", "const float m = orc_bf16_to_f32(xg[i]);"),
    "quant_no_floor": ("if (a < 0x1p-64f) a = 0x1p-64f;", ";"),
    "quant_group_stride": ("const uint16_t *xg = x + t * H + (int64_t)q * g;", "const uint16_t *xg = x + t * H + q;"),
    "quant_amax_skips_last": ("for (int32_t i = 0; i < g; ++i) {\n                const float m",
                              "for (int32_t i = 0; i < g - 1; ++i) {\n                const float m"),
    "dequant_scale_index": ("scales[t * num_scales + i / g]", "scales[t * num_scales + i % num_scales]"),
    "dequant_scale_dropped": ("out[t * H + i] = orc_f32_to_bf16_rne(v * scales[t * num_scales + i / g]);",
                              "out[t * H + i] = orc_f32_to_bf16_rne(v);"),
    "rdma_prefix_skips_node_first_rank": (
        "for (int32_t r = n * 8; r < R && r < (n + 1) * 8; ++r)\n                    any |= is_token_in_rank[t * R + r] != 0;",
        "for (int32_t r = n * 8 + 1; r < R && r < (n + 1) * 8; ++r)\n                    any |= is_token_in_rank[t * R + r] != 0;"),
    "rdma_prefix_not_cumulative": ("running += any;", "running = any;"),
    "gbl_counts_rank0_column": ("running += is_token_in_rank[t * R + r] != 0;", "running += is_token_in_rank[t * R] != 0;"),
    "recv_rdma_prefix_exclusive": ("sum += num_tokens_per_rdma_rank[n];\n        recv_rdma_rank_prefix_sum[n] = sum;",
                                   "recv_rdma_rank_prefix_sum[n] = sum;\n        sum += num_tokens_per_rdma_rank[n];"),
    "num_recv_is_last_rank": ("*num_recv_tokens = sum;", "*num_recv_tokens = num_tokens_per_rank[R - 1];"),
    "notify_rank_count_unchecked": ("if (running != num_tokens_per_rank[r]) status |= ORC_COUNT_MISMATCH;", ";"),
    "notify_node_count_unchecked": ("if (running != num_tokens_per_rdma_rank[n]) status |= ORC_COUNT_MISMATCH;", ";"),
    "overflow_row_not_advanced": ("status |= ORC_RECV_OVERFLOW;\n                    ++row;\n                    continue;",
                                  "status |= ORC_RECV_OVERFLOW;\n                    continue;"),
    "bad_topk_not_flagged": ("        *status |= ORC_BAD_TOPK_IDX;\n        return 0;", "        return 0;"),
    "combine_bad_slot_not_flagged": (
        "            if (s < -1 || s >= num_recv) {\n                status |= ORC_BAD_SEND_SLOT;\n                continue;\n"
        "            }\n            float W = 0.0f;",
        "            if (s < -1 || s >= num_recv) {\n                continue;\n            }\n            float W = 0.0f;"),
    "combine_slot_bound_inclusive": (
        "            if (s < -1 || s >= num_recv) {\n                status |= ORC_BAD_SEND_SLOT;\n                continue;\n"
        "            }\n            float W = 0.0f;",
        "            if (s < -1 || s > num_recv) {\n                status |= ORC_BAD_SEND_SLOT;\n                continue;\n"
        "            }\n            float W = 0.0f;"),
    "combined_weights_not_cleared": (
        "        if (combined_topk_weights)\n            for (int32_t j = 0; j < K; ++j) combined_topk_weights[t * K + j] = 0.0f;",
        ""),
    "combine_acc_not_cleared": ("        for (int32_t i = 0; i < H; ++i) acc_scratch[i] = 0.0f;", ""),
    "group_bad_id_not_flagged": (
        "if (i < last * K && (recv_topk_idx[i] < -1 || recv_topk_idx[i] >= er)) status |= ORC_BAD_TOPK_IDX;", ";"),
    "group_reads_slack_ids": (
        "if (i < last * K && (recv_topk_idx[i] < -1 || recv_topk_idx[i] >= er)) status |= ORC_BAD_TOPK_IDX;",
        "if ((recv_topk_idx[i] < -1 || recv_topk_idx[i] >= er)) status |= ORC_BAD_TOPK_IDX;"),
    "group_overflow_not_flagged": ("                        status |= ORC_RECV_OVERFLOW;\n                        continue;",
                                   "                        continue;"),
    "recv_idx_unmasked": ("recv_topk_idx[row * K + j] = on_r ? e - (int64_t)r * experts_per_rank : -1;",
                          "recv_topk_idx[row * K + j] = e - (int64_t)r * experts_per_rank;"),
    "fp8_scales_of_row": ("recv_x_scales[row * num_scales + i] = x_scales[t * num_scales + i];",
                          "recv_x_scales[row * num_scales + i] = x_scales[(row % T) * num_scales + i];"),
    "group_padding_x_not_zeroed": ("memset(grouped_x + pos * row_bytes, 0, (size_t)row_bytes);", ";"),
    "group_padding_scales_not_zeroed": (
        "for (int32_t s = 0; s < num_scales; ++s) grouped_x_scales[pos * num_scales + s] = 0.0f;", ";"),
    "group_padding_weight_not_zeroed": ("                grouped_weights[pos] = 0.0f;", ";"),
    "group_slot_pos_not_reset": ("        slot_pos[i] = -1;", ";"),
    "cached_scales_not_copied": (
        "for (int32_t i = 0; i < num_scales; ++i) recv_x_scales[s * num_scales + i] = x_scales[t * num_scales + i];",
        ";"),
    "e4m3_decode_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "quant_codes_group_stride": ("codes[t * H + (int64_t)q * g + i] = orc_e4m3_rne(v);",
                                 "codes[t * H + i] = orc_e4m3_rne(v);"),
    "weights_of_slot0": ("recv_topk_weights[row * K + j] = on_r ? topk_weights[t * K + j] : 0.0f;",
                         "recv_topk_weights[row * K + j] = on_r ? topk_weights[t * K] : 0.0f;"),
}

CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, pins
    from combine_ep_get_02_amd import inputs
    o = oracle.Oracle(oracle.load({lib!r}))
    checks = [lambda: pins.pin_golden(o), lambda: pins.pin_bf16_rounding(o),
              lambda: pins.pin_workload(o, inputs.generate("tiny")),
              lambda: pins.pin_workload(o, inputs.generate("sweep"), hidden=64),
              lambda: pins.pin_fp8_and_cached(o, inputs.generate("tiny")),
              lambda: pins.pin_golden_grouping(o), lambda: pins.pin_group_by_expert(o, inputs.generate("tiny"), 4),
              lambda: pins.pin_group_by_expert(o, inputs.generate("sweep"), 1, hidden=32),
              lambda: pins.pin_dispatch_prefix_checks(o, inputs.generate("tiny")),
              lambda: pins.pin_count_checks_and_overflow(o, inputs.generate("sweep")), lambda: pins.pin_flags(o),
              lambda: pins.pin_bruteforce(o), lambda: pins.pin_e4m3(o), lambda: pins.pin_quantize(o)]
    errs = []
    for check in checks:  # in order, stopping at the first pin that fails
        errs = check()
        if errs:
            break
    print("CAUGHT" if errs else "MISSED", errs[:2])
""")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    import oracle

    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique/present"
    mut_c = tmp_path / "mutant.c"
    mut_c.write_text(src.replace(before, after))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(mut_c), lib)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    # caught: a pin failed, or the mutant crashed the child on a signal; a Python
    # exception inside the pins would be a broken pin, not a catch.
    caught = "CAUGHT" in p.stdout or p.returncode < 0
    assert caught, f"mutant {name} passed every pin: {p.stdout[-500:]} {p.stderr[-500:]}"
