"""The pins catch planted mistakes in the oracle.

Each case copies oracle.c, plants one plausible mistake in the copy (a
dropped term, a wrong operand or index, a reversed tie-break, a missing
scale), builds it into a library of its own and routes the oracle through it
while a chosen set of pins from test_oracle_pins runs. At least one of those
pins must fail. The planted text must occur exactly once in oracle.c, so a
change to the oracle that moves it fails here loudly instead of testing
nothing. CPU only; the GPU library is not involved.
"""
from __future__ import annotations

import os

import pytest

import oracle
import test_oracle_pins as pins

# (name, text in oracle.c, replacement, pins that must notice)
MUTANTS = [
    ("indexer: weight applied before the ReLU",
     "double relu = dot > 0.0 ? dot : 0.0;\n"
     "        total += (double)w[(int64_t)b * H + h] * relu;",
     "double wd = (double)w[(int64_t)b * H + h] * dot;\n"
     "        total += wd > 0.0 ? wd : 0.0;",
     [pins.test_indexer_relu_before_weight]),
    ("indexer: last head dropped",
     "for (int h = 0; h < H; ++h) {",
     "for (int h = 0; h < H - 1; ++h) {",
     [pins.test_indexer_single_head_is_relu_of_matmul,
      pins.test_indexer_weight_scaling_and_head_permutation,
      pins.test_indexer_mt_equals_fp64_einsum]),
    ("indexer: a token reads the keys of the wrong batch row",
     "const uint16_t* krow = k + ((int64_t)(b / T) * N + j) * D;",
     "const uint16_t* krow = k + ((int64_t)(b % B) * N + j) * D;",
     [pins.test_indexer_mt_equals_fp64_einsum,
      pins.test_indexer_mt_token_equals_the_single_token_indexer]),
    ("top-k: ties broken towards the larger index",
     "return (a->i > b->i) - (a->i < b->i);",
     "return (a->i < b->i) - (a->i > b->i);",
     [lambda: pins.test_topk_matches_rank_definition(0), pins.test_topk_special_rows]),
    ("top-k: smallest values selected",
     "if (a->v > b->v) return -1;\n  if (a->v < b->v) return 1;",
     "if (a->v < b->v) return -1;\n  if (a->v > b->v) return 1;",
     [lambda: pins.test_topk_matches_rank_definition(1), pins.test_topk_invariants_and_torch_values]),
    ("top-k: ragged lengths ignored",
     "const int n = lengths[b];",
     "const int n = N;",
     [lambda: pins.test_topk_ragged_matches_rank_definition_of_the_prefix(0)]),
    ("attention: softmax scale dropped",
     "z[r] = scale * dot;",
     "z[r] = dot;",
     [pins.test_attend_dense_equals_sdpa, pins.test_attend_closed_forms]),
    ("attention: window rows left out",
     "const int R = k + W;",
     "const int R = k;",
     [pins.test_attend_sparse_with_window_equals_sdpa_on_gathered_rows,
      pins.test_attend_window_rows_equal_selected_rows_and_permutation]),
    ("attention: a token gathers the wrong batch row's keys",
     "r < k ? kv + ((int64_t)(b / T) * N + idx[(int64_t)b * k + r]) * D",
     "r < k ? kv + ((int64_t)(b % B) * N + idx[(int64_t)b * k + r]) * D",
     [pins.test_attend_mt_equals_sdpa_per_token]),
    ("attention: the sink left out of the denominator",
     "double l = sink ? exp(sink[h] - m) : 0.0;",
     "double l = 0.0;",
     [pins.test_attend_sink_equals_sdpa_with_a_zero_value_row, pins.test_attend_sink_closed_forms]),
    ("compressor: weights not normalised",
     "acc += (a[i] / l) * bf16_value(rows[(int64_t)i * D + d]);",
     "acc += a[i] * bf16_value(rows[(int64_t)i * D + d]);",
     [pins.test_compress_closed_forms, pins.test_compress_equals_torch_softmax_gate]),
    ("compressor: every gate score taken from the group's first row",
     "dot += (double)wg[d] * bf16_value(rows[(int64_t)i * D + d]);",
     "dot += (double)wg[d] * bf16_value(rows[d]);",
     [pins.test_compress_equals_torch_softmax_gate, pins.test_compress_closed_forms]),
    ("query projection: weight read transposed",
     "acc += bf16_value(xrow[i]) * bf16_value(wrow[i]);",
     "acc += bf16_value(xrow[i]) * bf16_value(w[(int64_t)i * O + o]);",
     [pins.test_qproj_equals_fp64_matmul, pins.test_qproj_one_hot_and_scaling_are_exact]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, checks):
    src = open(oracle.source_path(), encoding="utf-8").read()
    assert src.count(old) == 1, f"{name}: the planted text must occur once in oracle.c"
    mutant_c = os.path.join(tmp_path, "oracle_mutant.c")
    with open(mutant_c, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_source(mutant_c, os.path.join(tmp_path, "liboracle_mutant.so"))
    caught = []
    with oracle.using_library(lib):
        for check in checks:
            try:
                check()
            except (AssertionError, ValueError) as exc:  # a failed pin, or a rejected result
                caught.append(f"{getattr(check, '__name__', 'check')}: {type(exc).__name__}")
    assert caught, f"no pin noticed the planted mistake: {name}"


def test_unaltered_copy_passes_the_same_pins(tmp_path):
    # The harness itself: a rebuilt, unaltered copy passes every pin used above.
    lib = oracle.compile_source(oracle.source_path(), os.path.join(tmp_path, "liboracle_copy.so"))
    with oracle.using_library(lib):
        for _, _, _, checks in MUTANTS:
            for check in checks:
                check()
