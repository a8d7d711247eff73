"""Planted mistakes in the oracle must fail at least one pin.

Each mutant edits one passage of oracle.c (on the CPU, in a temporary copy), builds
it, and runs every pin of oracle_pins.py against that build in a child process (a
mutant that reads out of bounds may crash; that also counts as caught).  The list
covers the pitfall table of "Paged attention for decode in C" (section 5) where it
applies to a two-pass oracle, the printed phase-2 form of the PagedAttention V2 page,
and the merge edge cases of MergeAttnStates.
"""
import json
import os
import subprocess
import sys

import pytest

from oracle import oracle as oracle_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (text in oracle.c, replacement).  Pitfall s13 (accepting an empty context) is
# not listed: a decode query at position n - 1 = -1 is also refused by the position
# rule, so dropping the length check alone changes nothing (an equivalent mutant).
MUTANTS = {
    # decode page, section 5
    "s03_logical_index_as_block_id": ("int64_t block_id = table[j / block_size];",
                                      "int64_t block_id = j / block_size;"),
    "s04_no_kv_head_offset": ("int64_t base = (slot * num_kv_heads + g) * head_dim;",
                              "int64_t base = (slot * num_kv_heads) * head_dim;"),
    "s05_round_robin_heads": ("for (int h = g * group; h < (g + 1) * group; ++h)",
                              "for (int h = g; h < job->num_heads; h += P->num_kv_heads)"),
    "s06_window_of_w_plus_1": ("s = e - job->sliding_window;", "s = e - job->sliding_window - 1;"),
    "s07_query_at_n": ("pos[s] = seq_lens[s] - 1;", "pos[s] = seq_lens[s];"),
    "s08_v_from_k_slab": ("gather_head(P->v, P->dtype", "gather_head(P->k, P->dtype"),
    "s14_trust_max_blocks": ("if (need > job->max_blocks) return ORC_EINVAL;", ""),
    "s15_trust_block_ids": ("if (table[i] < 0 || table[i] >= P->num_blocks) return ORC_EINVAL;", ""),
    # phase 2 of the PagedAttention V2 page as printed: un-normalised partition outputs
    "unnormalised_partition_outputs": (
        "memcpy(job->tmp_out + idx * P->dv, orow, sizeof(double) * (size_t)P->dv);",
        "for (int d = 0; d < P->dv; ++d) job->tmp_out[idx * P->dv + d] = orow[d] * l;"),
    "reduce_without_rescale": ("double w = exp_sums[base + p] * exp(max_logits[base + p] - M);",
                               "double w = exp_sums[base + p];"),
    # arithmetic slips
    "scale_dropped": ("s[j - lo] = scale * dot + slope", "s[j - lo] = dot + slope"),
    "causal_excludes_self": ("int64_t e = job->causal ? (int64_t)job->positions[t] + 1 : n;",
                             "int64_t e = job->causal ? (int64_t)job->positions[t] : n;"),
    "lse_without_max": ("return l > 0.0 ? m + log(l) : -INFINITY;", "return l > 0.0 ? log(l) : -INFINITY;"),
    "no_final_normalisation": ("double inv = 1.0 / l;", "double inv = 1.0;"),
    "f16_exponent_bias": ("mag = ldexp((double)(1024 + f), e - 25);", "mag = ldexp((double)(1024 + f), e - 24);"),
    "bf16_wrong_shift": ("uint32_t bits = (uint32_t)h << 16;", "uint32_t bits = (uint32_t)h << 15;"),
    "write_kv_row_is_token": ("int64_t row = block_id * block_size + offset;", "int64_t row = t;"),
    # the merge of two states (MergeAttnStates) and its edge rules
    "merge_keeps_plus_inf": ("return isinf(x) ? -INFINITY : (double)x;", "return (double)x;"),
    "merge_both_ninf_emits_suffix": (
        "out[row + d] = load_elem(prefix_out, dtype, row + d);\n        merged = -INFINITY;",
        "out[row + d] = load_elem(suffix_out, dtype, row + d);\n        merged = -INFINITY;"),
    "merge_pass_through_off_by_one": ("t >= prefill_tokens_with_context;", "t > prefill_tokens_with_context;"),
    "merge_swapped_weights": ("out[row + d] = wa * load_elem(prefix_out", "out[row + d] = wb * load_elem(prefix_out"),
    "merge_lse_is_the_larger": ("return big + log1p(exp(small - big));", "return big;"),
    "merge_lse_log_not_log1p": ("return big + log1p(exp(small - big));", "return big + log(exp(small - big));"),
    # the two-pass core on caller-gathered arrays (MlaPrefillAttention), and the row
    # mask of the varlen oracle
    "gathered_out_stride_dk": ("s, out + r * dv, &m, &l);", "s, out + r * dk, &m, &l);"),
    "gathered_q_stride_dv": ("attend(q + r * dk, K, V, dk, dv, lo[r]", "attend(q + r * dv, K, V, dk, dv, lo[r]"),
    "gathered_lo_ignored": ("dk, dv, lo[r], hi[r], scale", "dk, dv, 0, hi[r], scale"),
    "gathered_hi_exclusive_off_by_one": ("dk, dv, lo[r], hi[r], scale", "dk, dv, lo[r], hi[r] - 1, scale"),
    "gathered_range_unchecked": ("if (lo[r] < 0 || hi[r] > n_keys) return ORC_EINVAL;", "if (lo[r] < 0 || hi[r] > n_keys) {}"),
    "row_mask_inverted": ("return job->row_mask == NULL || job->row_mask[t * job->num_heads + h];",
                          "return job->row_mask == NULL || !job->row_mask[t * job->num_heads + h];"),
    "row_mask_head_major": ("return job->row_mask == NULL || job->row_mask[t * job->num_heads + h];",
                            "return job->row_mask == NULL || job->row_mask[(int64_t)h * job->num_tokens + t];"),
    "row_mask_ignored": ("return job->row_mask == NULL || job->row_mask[t * job->num_heads + h];", "return 1;"),
    # attention sinks (ForwardWithSinks)
    "sink_left_out_of_max": ("  double m = sink;\n", "  double m = -INFINITY;\n"),
    "sink_left_out_of_sum": ("double l = sink == -INFINITY ? 0.0 : exp(sink - m);", "double l = 0.0;"),
    "sink_counted_per_partition": (
        "attend(qrow, K, V, P->dk, P->dv, lo, hi, job->scale, -INFINITY, slope, ref, sc, orow, &m, &l);",
        "attend(qrow, K, V, P->dk, P->dv, lo, hi, job->scale, job->sinks ? job->sinks[h] : -INFINITY, slope, ref, sc, "
        "orow, &m, &l);"),
    "reduce_without_sink": ("double total = sink == -INFINITY ? 0.0 : exp(sink - M);", "double total = 0.0;"),
    # encoders and the latent-cache gather (GatherMlaCache)
    "half_rounds_toward_zero": ("double r = nearbyint(ldexp(m, 11));", "double r = trunc(ldexp(m, 11));"),
    "half_subnormal_truncates": ("(uint16_t)nearbyint(ldexp(a, 24))", "(uint16_t)trunc(ldexp(a, 24))"),
    "bf16_truncates": ("u += 0x7fffu + ((u >> 16) & 1u);", ""),
    "bf16_ties_away": ("u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "gather_ignores_seq_starts": ("int64_t pos = t - cu_seq_lens[b] + (seq_starts ? seq_starts[b] : 0);",
                                  "int64_t pos = t - cu_seq_lens[b];"),
    "gather_slot_is_block_index": ("int64_t idx = pos / block_size, slot = pos % block_size;",
                                   "int64_t idx = pos / block_size, slot = idx % block_size;"),
    "gather_copies_rows_past_end": ("if (t >= cu_seq_lens[b + 1]) continue;", ""),
    "gather_trusts_block_ids": ("if (block < 0 || block >= num_blocks) return ORC_EINVAL;", ""),
    # fp8 (E4M3) caches and the per-tensor K / V scales
    "e4m3_bias_8": ("mag = ldexp((double)(8 + f), e - 10);", "mag = ldexp((double)(8 + f), e - 11);"),
    "e4m3_subnormal_as_normal": ("mag = ldexp((double)f, -9);", "mag = ldexp((double)(8 + f), -10);"),
    "e4m3_nan_as_largest": ("else if (e == 15 && f == 7)\n    mag = NAN;", "else if (e == 16)\n    mag = NAN;"),
    "e4m3_exponent_15_is_nan": ("else if (e == 15 && f == 7)", "else if (e == 15)"),
    "e4m3_sign_ignored": ("  return sign ? -mag : mag;\n}\n\nstatic double load_elem",
                          "  return mag;\n}\n\nstatic double load_elem"),
    "k_scale_on_v": ("gather_head(P->v, P->dtype, P->v_scale", "gather_head(P->v, P->dtype, P->k_scale"),
    "v_scale_dropped": ("gather_head(P->v, P->dtype, P->v_scale", "gather_head(P->v, P->dtype, 1.0"),
    "scale_divides": ("load_elem(pool, dtype, base + d) * scale;", "load_elem(pool, dtype, base + d) / scale;"),
    # ALiBi (v2 page, phase 1), counted from the row's last visible position
    "alibi_sign": ("s[j - lo] = scale * dot + slope * (double)(j - ref);",
                   "s[j - lo] = scale * dot - slope * (double)(j - ref);"),
    "alibi_absolute_position": ("s[j - lo] = scale * dot + slope * (double)(j - ref);",
                                "s[j - lo] = scale * dot + slope * (double)j;"),
    "alibi_ref_is_end": ("const int64_t ref = end - 1;", "const int64_t ref = end;"),
    "alibi_slope_of_kv_head": ("const double slope = job->alibi ? job->alibi[h] : 0.0;",
                               "const double slope = job->alibi ? job->alibi[g] : 0.0;"),
    "alibi_partition_relative": (
        "attend(qrow, K, V, P->dk, P->dv, lo, hi, job->scale, -INFINITY, slope, ref, sc, orow, &m, &l);",
        "attend(qrow, K, V, P->dk, P->dv, lo, hi, job->scale, -INFINITY, slope, hi - 1, sc, orow, &m, &l);"),
    "scales_unchecked": ("  if (!isfinite(P->k_scale) || !(P->k_scale > 0.0) || !isfinite(P->v_scale) || !(P->v_scale > 0.0))\n    return ORC_EINVAL;\n", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle_mod.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutant {name}: passage not found in oracle.c"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle_mod.build(str(mutated), lib)
    code = f"import sys; sys.path.insert(0, {ROOT!r}); from tests import oracle_pins; oracle_pins.run_all({lib!r})"
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    if proc.returncode != 0:
        return  # crashed: caught
    lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
    assert lines, proc.stdout + proc.stderr
    failed = json.loads(lines[-1])["failed"]
    assert failed, f"mutant {name} passed every pin"
