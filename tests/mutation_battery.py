"""Run the oracle's pins against another build of oracle.c.

    python tests/mutation_battery.py /path/to/liboracle_variant.so

Exits 0 if every pin passes, 1 if any fails (a planted mistake was caught).
Used by test_oracle_mutations.py, which runs it in a subprocess so that a
mutant that crashes cannot take the test run down with it.
"""
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import test_oracle_pins as P  # noqa: E402

BATTERY = [
    (P.test_1d_matches_torch_grouped_conv, (3, 7, 8, 4, False)),
    (P.test_1d_matches_torch_grouped_conv, (3, 7, 8, 4, True)),
    (P.test_1d_matches_torch_grouped_conv, (2, 50, 3, 15, False)),
    (P.test_1d_matches_torch_grouped_conv, (2, 13, 4, 2, True)),
    (P.test_1d_matches_im2col_matmul, (3, 9, 2, 9, True)),
    (P.test_1d_delta_kernels, (9, False)),
    (P.test_1d_delta_kernels, (5, True)),
    (P.test_1d_linearity_and_bias_superposition, ()),
    (P.test_1d_causality_and_batch_independence, ()),
    (P.test_1d_masked_frames_exact_zero_and_no_nan_leak, ()),
    (P.test_2d_matches_torch_grouped_conv, (2, 9, 8, 3, 3, 3, 2, 1)),
    (P.test_2d_matches_torch_grouped_conv, (2, 7, 9, 2, 3, 1, 2, 1)),
    (P.test_2d_matches_torch_grouped_conv, (1, 12, 4, 5, 5, 3, 3, 2)),
    (P.test_2d_center_delta_closed_form, ()),
    (P.test_2d_masked_rows_exact_zero_and_no_nan_leak, ()),
    (P.test_2d_asymmetric_pads_match_torch, (2, 9, 8, 3, 3, 3, 2, (2, 1, 2, 1))),
    (P.test_2d_asymmetric_pads_match_torch, (2, 12, 10, 2, 3, 3, 2, (1, 0, 0, 2))),
    (P.test_2d_causal_pads_never_look_ahead, ()),
    (P.test_2d_causal_present_tap_closed_form, ()),
    (P.test_bwd_asymmetric_pads_match_torch_autograd, (2, 9, 8, 3, 3, 3, 2, (2, 1, 2, 1))),
    (P.test_bwd_asymmetric_pads_match_torch_autograd, (2, 12, 10, 2, 3, 3, 2, (1, 0, 0, 2))),
    (P.test_bwd_matches_torch_autograd, (2, 9, 8, 3, 3, 3, 2, 1)),
    (P.test_bwd_matches_torch_autograd, (1, 12, 4, 5, 5, 3, 3, 2)),
    (P.test_bwd_adjoint_and_bilinear_identities, ()),
    (P.test_bwd_masks_and_no_nan_leak, ()),
    (P.test_front_matches_torch_chain, (3, 13, 9, 3)),
    (P.test_front_center_delta_closed_form, ()),
    (P.test_front_fully_masked_rows_equal_output_bias, ()),
    (P.test_front_input_is_not_length_masked, ()),
    (P.test_front_causal_matches_torch_chain, (3, 13, 9, 3)),
    (P.test_front_causal_present_tap_and_no_look_ahead, ()),
    (P.test_front_causal_empty_item_is_output_bias, ()),
    (P.test_front_causal_bwd_matches_torch_autograd, (3, 13, 9, 3)),
    (P.test_front_bwd_matches_torch_autograd, (2, 16, 12, 4)),
    (P.test_front_bwd_matches_torch_autograd, (3, 13, 9, 3)),
    (P.test_front_bwd_closed_forms_and_linearity, ()),
    (P.test_front_bwd_masked_input_rows_never_read, ()),
    (P.test_1d_bwd_matches_torch_autograd, (3, 7, 8, 4, True)),
    (P.test_1d_bwd_matches_torch_autograd, (2, 50, 3, 15, False)),
    (P.test_1d_bwd_adjoint_closed_forms_and_masks, ()),
    (P.test_1d_bwd_finite_differences_in_w, ()),
    (P.test_1d_stream_chunks_equal_the_whole_causal_conv, (4,)),
    (P.test_1d_stream_chunks_equal_the_whole_causal_conv, (9,)),
    (P.test_1d_stream_delta_kernels_read_the_cache, ()),
    (P.test_1d_stream_empty_chunk_keeps_the_cache_and_nan_past_length_never_read, ()),
]


def main(path, stop_at_first=True):
    oracle._lib = oracle._bind(path)
    failed = []
    for fn, args in BATTERY:
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure counts as a catch
            failed.append(f"{fn.__name__}{args}: {traceback.format_exc(limit=1).splitlines()[-1]}")
            if stop_at_first:
                break
    for f in failed:
        print("caught by", f)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
