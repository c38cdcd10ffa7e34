"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins in test_oracle_pins.py catch every one of them.

Each mutation is a textual edit of moelora_ref.c compiled to a temporary
library; the unmodified oracle is never touched.
"""
import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = {
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "gate_up_swapped": ("h[i] = silu(g[i]) * g[(size_t)I + i];",
                        "h[i] = silu(g[(size_t)I + i]) * g[i];"),
    "gate_up_expand_dropped": ("g[n] += acc;", "g[n] += 0.0 * acc;"),
    "down_expand_dropped": ("y[m] += acc;", "y[m] += 0.0 * acc;"),
    "b_gu_transposed": ("acc += z[c] * ld(B_gu, brow + c, dtype);",
                        "acc += z[c] * ld(B_gu, pair * I2 * r + (size_t)c * I2 + n, dtype);"),
    "a_d_row_stride_H": ("size_t arow = (pair * r + c) * I;",
                         "size_t arow = (pair * r + c) * H;"),
    "w_gu_transposed": ("ldw(W_gu, s_gu, fp8, wrow, (size_t)H, (size_t)c, dtype)",
                        "ldw(W_gu, s_gu, fp8, (size_t)e * H + c, I2, n, dtype)"),
    "fp8_scale_of_wrong_row": ("return (double)scale[row] * fp8[",
                               "return (double)scale[row ^ 1] * fp8["),
    "fp8_exponent_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                            "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_subnormals_as_normals": ("if (e == 0)\n        v = ldexp((double)m / 8.0, -6);",
                                  "if (e == 0)\n        v = ldexp(1.0 + (double)m / 8.0, -7);"),
    "no_renormalise": ("w[(size_t)t * k + j] = prob[ids[(size_t)t * k + j]] / kept;",
                       "w[(size_t)t * k + j] = prob[ids[(size_t)t * k + j]];"),
    "ties_to_higher_index": ("(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    "weight_of_wrong_expert": ("double wj = w[(size_t)t * k + j];",
                               "double wj = w[(size_t)t * k + (k - 1 - j)];"),
    "no_block_padding": ("seg_start[e + 1] = seg_start[e] + (c + BM - 1) / BM * BM;",
                         "seg_start[e + 1] = seg_start[e] + c;"),
    "tile_length_off_by_one": ("tiles[4 * nt + 3] = hi - lo;", "tiles[4 * nt + 3] = hi - lo + (b > 0);"),
    "base_rows_first": ("((adapter_ids && adapter_ids[(p) / k] >= 0 && adapter_ids[(p) / k] < NA) \\\n         ? adapter_ids[(p) / k]",
                        "((adapter_ids && adapter_ids[(p) / k] >= 0 && adapter_ids[(p) / k] < NA) \\\n         ? (adapter_ids[(p) / k] + 1) % (NA + 1)"),
}

PIN_CALLS = [
    (pins.test_golden_hand_example, {}),
    (pins.test_golden_route_cases, {}),
    (pins.test_route_matches_stable_sort_and_softmax, dict(T=40, E=32, k=4)),
    (pins.test_align_matches_bruteforce, dict(T=37, k=2, E=5, NA=3, BM=4)),
    (pins.test_align_matches_bruteforce, dict(T=64, k=2, E=8, NA=16, BM=16)),
    (pins.test_dense_ffn_is_textbook, {}),
    (pins.test_grouped_equals_dense, dict(seed=1)),
    (pins.test_single_adapter_equals_merged_weights, {}),
    (pins.test_identical_experts_make_routing_irrelevant, {}),
    (pins.test_fp8_e4m3_codes_match_the_format, {}),
    (pins.test_fp8_weights_equal_bf16_dequantised_weights, {}),
    (pins.test_fp8_weights_against_dense_float64, {}),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = oracle.source()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    caught = []
    for fn, kw in PIN_CALLS:
        try:
            fn(variant, **kw)
        except (AssertionError, ValueError):
            caught.append(fn.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_all_pins(tmp_path):
    variant = oracle.build_variant(oracle.source(), str(tmp_path / "copy.so"))
    for fn, kw in PIN_CALLS:
        fn(variant, **kw)
