"""Plants plausible mistakes in the oracle's C source and checks that each one
makes at least one pin fail (so the pins would have caught it).  CPU only; the
mutants are compiled into a temporary directory and never touch the oracle
that the other tests use."""
import os

import pytest

import pins
from oracle import pa_ref

# (name, exact snippet in pa_ref.c, mistaken replacement).  Every mutant keeps
# the oracle's reads inside its buffers (a mistake that reads out of bounds
# would crash the test process rather than fail a pin).
MUTANTS = [
    ("gqa_modulo", "const int g = h / group;", "const int g = h % Hkv;"),
    ("slot_shift", "int slot = tok % bs;\n        const int64_t krow",
     "int slot = (tok + 1) % bs;\n        const int64_t krow"),
    ("causal_off_by_one", "if (P->mask == REF_MASK_CAUSAL && prefix + i + 1 < hi)\n        hi = prefix + i + 1;",
     "if (P->mask == REF_MASK_CAUSAL && prefix + i < hi)\n        hi = prefix + i;"),
    ("causal_always", "if (P->mask == REF_MASK_CAUSAL && prefix + i + 1 < hi)",
     "if (prefix + i + 1 < hi)"),
    ("band_left_off_by_one", "if (pos - P->win_left > lo)\n            lo = pos - P->win_left;",
     "if (pos - P->win_left + 1 > lo)\n            lo = pos - P->win_left + 1;"),
    ("band_right_ignored", "if (pos + 1 + P->win_right < hi)\n            hi = pos + 1 + P->win_right;",
     "if (pos + 1 < hi)\n            hi = pos + 1;"),
    ("band_position_without_prefix", "const int64_t pos = (int64_t)prefix + i;", "const int64_t pos = i;"),
    ("band_right_one_short", "            hi = pos + 1 + P->win_right;", "            hi = pos + P->win_right;"),
    ("prefix_plus_one", "const int prefix = kv - qlen > 0 ? kv - qlen : 0;",
     "const int prefix = kv - qlen + 1 > 0 ? kv - qlen + 1 : 0;"),
    ("no_scale", "z[j] = P->scale * dot;", "z[j] = dot;"),
    ("lse_no_log", "*lse = zmax + log(wsum);", "*lse = zmax + wsum;"),
    ("kv_layout_bhsd", "const int64_t krow = (((int64_t)phys * bs + slot) * Hkv + g) * Dk;",
     "const int64_t krow = (((int64_t)phys * Hkv + g) * bs + slot) * Dk;"),
    ("v_layout_bhsd", "const int64_t vrow = (((int64_t)phys * bs + slot) * Hkv + g) * vstride;",
     "const int64_t vrow = (((int64_t)phys * Hkv + g) * bs + slot) * vstride;"),
    ("mean_not_softmax", "o[e] /= wsum;", "o[e] /= (double)n;"),
    ("row_offset_dropped", "const int64_t t = P->row_start[b] + i;", "const int64_t t = i;"),
    ("q_head_is_kv_head", "const uint16_t *q = P->query + (t * H + h) * (int64_t)Dk;",
     "const uint16_t *q = P->query + (t * H + g) * (int64_t)Dk;"),
    ("f16_exponent_bias", "v = ldexp((double)(1024 + frac), expo - 25);",
     "v = ldexp((double)(1024 + frac), expo - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = ((uint32_t)b << 16) | 0x8000u;"),
    ("table_row_stride",
     "int32_t phys = P->block_tables[(int64_t)b * P->max_num_blocks_per_seq + tok / bs];\n        if (phys < 0",
     "int32_t phys = P->block_tables[(int64_t)b * (P->max_num_blocks_per_seq - 1) + tok / bs];\n        if (phys < 0"),
    ("v_uses_first_token", "o[e] += z[j] * elem(vsrc, vrow + e, P->dtype);",
     "o[e] += z[j] * elem(vsrc, vrow - (int64_t)slot * Hkv * vstride + e, P->dtype);"),
    ("shared_v_row_stride", "const int vstride = P->value_cache ? Dv : Dk;", "const int vstride = Dv;"),
    ("shared_v_last_columns", "const uint16_t *vsrc = P->value_cache ? P->value_cache : P->key_cache;",
     "const uint16_t *vsrc = P->value_cache ? P->value_cache : P->key_cache + (Dk - Dv);"),
    ("exp_without_shift_in_lse", "*lse = zmax + log(wsum);", "*lse = log(wsum);"),
    ("sparse_causal_ignored", "if (list && (tok < 0 || tok >= kv || tok > prefix + i)) {",
     "if (list && (tok < 0 || tok >= kv)) {"),
    ("sparse_causal_off_by_one", "if (list && (tok < 0 || tok >= kv || tok > prefix + i)) {",
     "if (list && (tok < 0 || tok >= kv || tok >= prefix + i)) {"),
    ("sparse_list_of_head_0", "list = P->topk_idx + (t * Hkv + g) * (int64_t)P->topk;",
     "list = P->topk_idx + (t * Hkv) * (int64_t)P->topk;"),
    ("tensor_bias_subtracted", "z[j] += from_f16_bits(P->mask_tensor", "z[j] -= from_f16_bits(P->mask_tensor"),
    ("tensor_transposed", "P->mask_tensor[(int64_t)i * REF_MASK_DIM + c]", "P->mask_tensor[(int64_t)c * REF_MASK_DIM + i]"),
    ("tensor_columns_not_shifted", "const int64_t c = (int64_t)tok - prefix;", "const int64_t c = (int64_t)tok;"),
    ("tensor_all_visible_outside", "else if (c > i)\n                z[j] = -INFINITY;", "else if (0)\n                z[j] = -INFINITY;"),
]


def test_mutant_snippets_are_unique():
    src = open(pa_ref.SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(pa_ref.SRC).read()
    assert src.count(old) == 1
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = pa_ref.build(str(path), str(tmp_path / f"libmut_{name}.so"))
    lib = pa_ref.load(lib_path)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            break   # one pin that fails is enough
    assert caught, f"mutant {name} passes every pin"
