"""The oracle's pins are sharp: each plausible mistake planted in a copy of the
oracle source (CPU only, compiled into a temp dir) makes at least one pin fail.

Every mutation keeps all memory accesses in bounds, so a mutant fails by
giving wrong numbers, never by crashing the test process.
"""
import os
import tempfile

import pytest

import oracle
from tests import test_oracle_alibi as ALIBI
from tests import test_oracle_fp8 as FP8
from tests import test_oracle_lse as LSE
from tests import test_oracle_mq as MQ
from tests import test_oracle_pins as PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "paged_decode_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("gqa_mapping_modulo", "int32_t h = kh * G + g;", "int32_t h = g * pr->KH + kh;"),
    ("query_indexed_by_kv_head", "dot += query_at(pr, r, h, d)", "dot += query_at(pr, r, kh, d)"),
    ("key_layout_token_major",
     "int64_t idx = ((((int64_t)b * pr->KH + kh) * (pr->D / x) + d / x) * pr->BS + o) * x + d % x;",
     "int64_t idx = ((((int64_t)b * pr->KH + kh) * pr->BS + o) * (pr->D / x) + d / x) * x + d % x;"),
    ("value_layout_token_major",
     "int64_t idx = (((int64_t)b * pr->KH + kh) * pr->D + d) * pr->BS + o;",
     "int64_t idx = (((int64_t)b * pr->KH + kh) * pr->BS + o) * pr->D + d;"),
    ("slot_off_by_one", "*slot = t % pr->BS;", "*slot = (t + 1) % pr->BS;"),
    ("scale_dropped", "score[t] = pr->scale * dot;", "score[t] = dot;"),
    ("softmax_sign", "double w = exp(score[t] - m);", "double w = exp(m - score[t]);"),
    ("partition_end_short", "int32_t t1 = t0 + pr->PS < L ? t0 + pr->PS : L;",
     "int32_t t1 = t0 + pr->PS - 1 < L ? t0 + pr->PS - 1 : L;"),
    ("partition_not_normalised", "for (int32_t d = 0; d < pr->D; ++d) o[d] /= l;", ""),
    ("sentinel_max_zero", "double m = -INFINITY, l = 0.0;", "double m = 0.0, l = 0.0;"),
    ("combine_drops_exp_sums", "Z += exp(ml[base + p] - Mx) * es[base + p];",
     "Z += exp(ml[base + p] - Mx);"),
    ("combine_weight_sign", "double w = exp(ml[base + p] - Mx) * es[base + p] / Z;",
     "double w = exp(Mx - ml[base + p]) * es[base + p] / Z;"),
    ("combine_floor_partitions", "int32_t n = (causal_len(seq_lens[s], M, mq) + PS - 1) / PS;",
     "int32_t n = causal_len(seq_lens[s], M, mq) / PS;"),
    ("binary16_bias", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);"),
    ("bfloat16_subnormal", "v = ldexp((double)f, -133);", "v = ldexp((double)f, -126);"),
    ("e4m3_bias", "v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 11);"),
    ("e4m3_exponent_15_is_nan", "} else if (e == 15 && f == 7) {", "} else if (e == 15) {"),
    ("e4m3_subnormal", "v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),
    ("k_scale_dropped", "return load_elem(pr->kc, idx, pr->kvdtype) * pr->kscale;",
     "return load_elem(pr->kc, idx, pr->kvdtype);"),
    ("v_scale_on_keys", "return load_elem(pr->kc, idx, pr->kvdtype) * pr->kscale;",
     "return load_elem(pr->kc, idx, pr->kvdtype) * pr->vscale;"),
    ("v_scale_dropped", "return load_elem(pr->vc, idx, pr->kvdtype) * pr->vscale;",
     "return load_elem(pr->vc, idx, pr->kvdtype);"),
    ("fp8_key_packing_8", "int32_t x = 16 / elem_size(pr->kvdtype);",
     "int32_t x = pr->kvdtype == ORACLE_FP8_E4M3 ? 8 : 16 / elem_size(pr->kvdtype);"),
    ("causal_off_by_one", "int32_t e = L - M + m + 1;", "int32_t e = L - M + m;"),
    ("causal_top_left", "int32_t e = L - M + m + 1;", "int32_t e = m + 1;"),
    ("query_row_ignores_token", "int64_t r = (int64_t)s * pr->M + mq;",
     "int64_t r = (int64_t)s * pr->M;"),
    ("query_decoded_as_cache", "(r * pr->H + h) * pr->D + d, pr->qdtype)",
     "(r * pr->H + h) * pr->D + d, pr->kvdtype)"),
    ("lse_drops_max", "pr->lse[r * pr->H + h] = m + log(l);", "pr->lse[r * pr->H + h] = log(l);"),
    ("lse_empty_zero", "pr->lse[r * pr->H + h] = -INFINITY;", "pr->lse[r * pr->H + h] = 0.0;"),
    ("merge_weight_sign", "double wa = exp(lse_a[r] - mx), wb = exp(lse_b[r] - mx);",
     "double wa = exp(mx - lse_a[r]), wb = exp(mx - lse_b[r]);"),
    ("merge_swapped_weights", "(wa * a[r * D + d] + wb * b[r * D + d]) / (wa + wb);",
     "(wb * a[r * D + d] + wa * b[r * D + d]) / (wa + wb);"),
    ("merge_unnormalised", "(wa * a[r * D + d] + wb * b[r * D + d]) / (wa + wb);",
     "(wa * a[r * D + d] + wb * b[r * D + d]);"),
    ("merge_lse_drops_max", "out_lse[r] = mx + log(wa + wb);", "out_lse[r] = log(wa + wb);"),
    ("merge_empty_lse_zero", "out_lse[r] = -INFINITY;", "out_lse[r] = 0.0;"),
    ("alibi_sign", "(double)pr->alibi[h] * (double)(t - (L0 - pr->M + mq));",
     "(double)pr->alibi[h] * (double)((L0 - pr->M + mq) - t);"),
    ("alibi_slope_by_kv_head", "(double)pr->alibi[h] * (double)(t - (L0 - pr->M + mq));",
     "(double)pr->alibi[kh] * (double)(t - (L0 - pr->M + mq));"),
    ("alibi_absolute_position", "(double)pr->alibi[h] * (double)(t - (L0 - pr->M + mq));",
     "(double)pr->alibi[h] * (double)t;"),
    ("alibi_query_at_sequence_end", "(double)pr->alibi[h] * (double)(t - (L0 - pr->M + mq));",
     "(double)pr->alibi[h] * (double)(t - (L0 - 1));"),
    ("alibi_before_scale",
     "score[t] = pr->scale * dot;\n            if (pr->alibi) /* the query sits at position "
     "L0 - M + mq */\n                score[t] += (double)pr->alibi[h] * (double)(t - (L0 - "
     "pr->M + mq));",
     "score[t] = dot;\n            if (pr->alibi) score[t] += (double)pr->alibi[h] * "
     "(double)(t - (L0 - pr->M + mq));\n            score[t] *= pr->scale;"),
]


def battery():
    """The pins, as plain calls; returns the names of those that fail."""
    checks = {
        "binary16": PINS.test_binary16_decoder_exhaustive,
        "bfloat16": PINS.test_bfloat16_decoder_exhaustive,
        "golden_uniform": PINS.test_golden_uniform_scores,
        "golden_argmax": PINS.test_golden_argmax_selection,
        "brute_force": lambda: PINS.test_brute_force_tiny("bf16", 4, 2, 16, 2),
        "library_dense": lambda: PINS.test_library_routine_dense("bf16", 8, 1, 64, 32, 0),
        "library_partitions": lambda: PINS.test_library_routine_partitions("bf16", 4),
        "partition_combine": lambda: PINS.test_partition_combine_equals_dense(32),
        "zero_length": PINS.test_zero_length_gives_zero_and_sentinels,
        "gather": PINS.test_gather_indices_brute_force,
        "e4m3": FP8.test_e4m3_decoder_exhaustive,
        "fp8_brute_force": lambda: FP8.test_fp8_brute_force_tiny("bf16", 4, 2, 16, 2),
        "fp8_library_dense": lambda: FP8.test_fp8_library_routine_dense("bf16", 8, 2, 128, 16, 0),
        "fp8_repacked": FP8.test_fp8_equals_repacked_fp32_cache,
        "mq_prefix": lambda: MQ.test_rows_equal_single_query_on_causal_prefix(2, "bf16"),
        "mq_library": lambda: MQ.test_library_routine_causal(3, 4),
        "mq_brute_force": MQ.test_brute_force_tiny,
        "lse_library": lambda: LSE.test_lse_matches_library_logsumexp("bf16", 1),
        "lse_merge_split": lambda: LSE.test_merge_of_disjoint_splits_is_full_attention("bf16", 4),
        "lse_merge_closed_form": LSE.test_merge_two_single_keys_closed_form,
        "lse_merge_identities": LSE.test_merge_infinite_identities_and_symmetry,
        "alibi_library": lambda: ALIBI.test_library_route("bf16", 3, 4),
        "alibi_closed_form": lambda: ALIBI.test_zero_query_closed_form(0.5),
        "alibi_steep": ALIBI.test_steep_slope_selects_the_query_position,
    }
    failed = []
    for name, fn in checks.items():
        try:
            fn()
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_battery():
    assert battery() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        csrc = os.path.join(d, f"{name}.c")
        with open(csrc, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.compile_source(csrc, os.path.join(d, f"{name}.so"))
        with oracle.using_library(lib):
            failed = battery()
    assert failed, f"no pin catches mutant {name}"
