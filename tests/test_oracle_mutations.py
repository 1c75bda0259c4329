"""Planted mistakes in the oracle are caught by the pins.

Each case copies the oracle's C source, applies one plausible mistake (a
dropped term, a wrong index or offset, a transposed operand, a wrong mask),
compiles the copy into a temporary library, runs every pin against it, and
requires at least one pin to fail. The mistakes are planted on the CPU only.
"""
import os

import pytest

import oracle
import pins

MUTATIONS = {
    "qk_drops_rope_dims": ("for (int d = 0; d < KV_DIM; ++d) dot +=",
                           "for (int d = 0; d < V_DIM; ++d) dot +="),
    "node_not_self_visible": ("for (int u = t; u != -1; u = parent_b[u]) visible[P + u] = 1;",
                              "for (int u = parent_b[t]; u != -1; u = parent_b[u]) visible[P + u] = 1;"),
    "only_direct_parent": ("for (int u = t; u != -1; u = parent_b[u]) visible[P + u] = 1;",
                           "for (int u = t, k = 0; u != -1 && k < 2; u = parent_b[u], ++k) visible[P + u] = 1;"),
    "tree_unmasked": ("for (int u = 0; u < T; ++u) visible[P + u] = 0;",
                      "for (int u = 0; u < T; ++u) visible[P + u] = 1;"),
    "first_prefix_key_dropped": ("for (int j = 0; j < P; ++j) visible[j] = 1;",
                                 "for (int j = 0; j < P; ++j) visible[j] = (j != 0);"),
    "segment_offset_wrong": ("for (int i = 0; i < b; ++i) seg += seq_lens[i];",
                             "for (int i = 0; i < b; ++i) seg += seq_lens[i] - T;"),
    "q_head_node_transposed": ("(((int64_t)b * T + t) * H + h) * KV_DIM",
                               "(((int64_t)b * H + h) * T + t) * KV_DIM"),
    "scale_applied_twice": ("scores[j] = sm_scale * dot;", "scores[j] = sm_scale * sm_scale * dot;"),
    "value_from_wrong_columns": ("out_row[d] += w * elem(kv_pool, vrow + d, f32);",
                                 "out_row[d] += w * elem(kv_pool, vrow + d + 64, f32);"),
    "f32_elements_swapped": ("if (f32) return (double)((const float*)base)[idx];",
                             "if (f32) return (double)((const float*)base)[idx ^ 1];"),
    "f32_read_as_bf16": ("if (f32) return (double)((const float*)base)[idx];",
                         "if (f32) return bf16_to_double(((const uint16_t*)base)[idx]);"),
    "bf16_widening_wrong": ("uint32_t u = ((uint32_t)bits) << 16;",
                            "uint32_t u = ((uint32_t)bits) << 15;"),
    "denominator_misses_tree": ("if (visible[j]) denom += exp(scores[j] - smax);",
                                "if (visible[j] && j < P) denom += exp(scores[j] - smax);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "libmutant.so"))
    orc = oracle.load(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
