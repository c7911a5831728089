"""Each plausible mistake planted in a copy of the oracle must fail some pin.

The copy is compiled on the CPU from the oracle source with one edit; the real
oracle is untouched.  Every edit keeps all memory accesses in bounds.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, [(text in pa_oracle.c, replacement), ...])
MUTANTS = [
    ("key_limit_off_by_one", [("if (!a->tree_mask) return t < L + i + 1;",
                               "if (!a->tree_mask) return t < L + i;")]),
    ("row_index_dropped", [("const int i = n - a->subsequence_begins[s];", "const int i = 0;")]),
    ("gqa_modulo_mapping", [("const int g = h / (Hq / Hkv);", "const int g = h % Hkv;")]),
    ("scale_dropped", [("z[t - lo] = a->scale * dot;", "z[t - lo] = dot;")]),
    ("window_one_short", [("lo = L + i + 1 - a->sliding_window;", "lo = L + i + 2 - a->sliding_window;")]),
    ("tree_bit_shifted", [("return j == i || ((a->tree_mask[n] >> j) & 1u);",
                           "return j == i || ((a->tree_mask[n] >> (j + 1)) & 1u);")]),
    ("tree_self_not_implied", [("return j == i || ((a->tree_mask[n] >> j) & 1u);",
                                "return ((a->tree_mask[n] >> j) & 1u);")]),
    ("tree_hides_the_past", [("if (t < L) return 1;", "if (t < L) return 0;")]),
    ("small_page_v_slot_major", [("if (bs < 16) return (size_t)d * bs + slot;",
                                  "if (bs < 16) return (size_t)slot * D + d;")]),
    ("small_page_k_d_major", [("if (bs < 16) return (size_t)slot * D + d;        /* small pages: [slot][d] */",
                               "if (bs < 16) return (size_t)d * bs + slot;")]),
    ("quantise_floor", [("float r = rintf(y);", "float r = floorf(y);")]),
    ("quantise_no_clamp", [("if (r > 255.0f) r = 255.0f;", "if (r > 255.0f) r = r - 256.0f;")]),
    ("quantise_zp_sign", [("zb = f32_to_f16(-mn / f16_to_f32(sb));", "zb = f32_to_f16(mn / f16_to_f32(sb));")]),
    ("quantise_scale_unrounded", [("const float s = f16_to_f32(sb), z = f16_to_f32(zb);",
                                   "const float s = range / 255.0f + (mx == mn), z = f16_to_f32(zb);")]),
    ("append_slot_shifted", [("const int slot = pos % bs;", "const int slot = (pos + 1) % bs;")]),
    ("append_scale_zp_swapped", [("sz[2 * srow + 0] = sb;", "sz[2 * srow + 0] = zb;"),
                                 ("sz[2 * srow + 1] = zb;", "sz[2 * srow + 1] = sb;")]),
    ("tree_first_row_mask", [("return j == i || ((a->tree_mask[n] >> j) & 1u);",
                              "return j == i || ((a->tree_mask[n - i] >> j) & 1u);")]),
    ("v_read_in_k_layout", [("const size_t vidx = page + v_offset(slot, d, D, u8, bs, a->page_layout);",
                             "const size_t vidx = page + k_offset(slot, d, D, u8, bs, a->page_layout);")]),
    ("k_page_row_major", [("page + k_offset(slot, d, D, u8, bs, a->page_layout), row);",
                           "page + (size_t)slot * D + d, row);")]),
    ("v_slot_quads_swapped", [("return ((((st * (D / 32) + d / 32) * 4 + qq) * 16 + d % 16) * 2 + (d % 32) / 16) * 4 + slot % 4;",
                               "return ((((st * (D / 32) + d / 32) * 4 + slot % 4) * 16 + d % 16) * 2 + (d % 32) / 16) * 4 + qq;")]),
    ("block_table_ignored", [("const size_t blk = (size_t)table[t / bs];",
                              "const size_t blk = (size_t)(t / bs);")]),
    ("slot_shifted", [("const int slot = t % bs;", "const int slot = (t + 1) % bs;")]),
    ("dequant_sign", [("[elem_idx] - zp) * s;", "[elem_idx] + zp) * s;")]),
    ("scale_zp_swapped", [("double s = dec_f16(p[2 * slot_idx + 0]);", "double s = dec_f16(p[2 * slot_idx + 1]);"),
                          ("double zp = dec_f16(p[2 * slot_idx + 1]);", "double zp = dec_f16(p[2 * slot_idx + 0]);")]),
    ("no_normalisation", [("for (int d = 0; d < D; ++d) out_row[d] /= Z;",
                           "for (int d = 0; d < D; ++d) out_row[d] /= 1.0;")]),
    ("softmax_temperature", [("const double w = exp(z[t - lo] - m);",
                              "const double w = exp(2.0 * (z[t - lo] - m));")]),
    ("f16_exponent_bias", [("v = ldexp((double)(man | 0x400), exp - 25);",
                            "v = ldexp((double)(man | 0x400), exp - 24);")]),
    ("f16_subnormal_scale", [("v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);")]),
    ("bf16_shift", [("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;")]),
    ("q_head_major_layout", [("const size_t q_off = ((size_t)n * Hq + h) * D;",
                              "const size_t q_off = ((size_t)h * a->num_tokens + n) * D;")]),
    ("k_dims_reversed", [("page + k_offset(slot, d, D, u8, bs, a->page_layout), row);",
                          "page + k_offset(slot, D - 1 - d, D, u8, bs, a->page_layout), row);")]),
    # the subset form (rows given as (token, q head) pairs); the indices are
    # reduced into range so the mistake stays in bounds
    ("pairs_token_head_swapped", [("n = a->pairs[2 * it];\n      h = a->pairs[2 * it + 1];",
                                   "n = a->pairs[2 * it + 1] % a->num_tokens;\n"
                                   "      h = a->pairs[2 * it] % a->num_q_heads;")]),
    ("rowmajor_v_read_d_major", [("static size_t v_offset(int slot, int d, int D, int u8, int bs, int layout) {\n  if (layout == 1) return (size_t)slot * D + d;",
                                  "static size_t v_offset(int slot, int d, int D, int u8, int bs, int layout) {\n  if (layout == 1) return (size_t)d * bs + slot;")]),
    ("rowmajor_ignored", [("static size_t k_offset(int slot, int d, int D, int u8, int bs, int layout) {\n  if (layout == 1) return (size_t)slot * D + d;",
                           "static size_t k_offset(int slot, int d, int D, int u8, int bs, int layout) {\n  if (layout == 9) return (size_t)slot * D + d;")]),
    ("pairs_first_item_only", [("n = a->pairs[2 * it];\n      h = a->pairs[2 * it + 1];",
                                "n = a->pairs[0];\n      h = a->pairs[1];")]),
]

PIN_ORDER = ["hand", "closed", "rows", "window", "gqa", "u8", "permutation", "ragged", "sdpa", "tree",
             "append", "pairs", "layout"]


def _source():
    with open(oracle.SRC) as f:
        return f.read()


def test_pin_list_is_complete():
    assert sorted(PIN_ORDER) == sorted(ALL_PINS)


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, edits):
    src = _source()
    for old, new in edits:
        assert old in src, f"mutation site for {name} not found in the oracle source"
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        orc = oracle.build_variant(src, d)
        caught = []
        for pin in PIN_ORDER:
            try:
                ALL_PINS[pin](orc)
            except (AssertionError, ValueError) as e:
                caught.append(pin)
                break
        assert caught, f"no pin catches the planted mistake {name}"
