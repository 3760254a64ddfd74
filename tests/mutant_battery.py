"""Run the oracle's pin checks against one build of the oracle source.

    python tests/mutant_battery.py path/to/liboracle_variant.so

Prints one JSON line {"checks": n, "failed": [...]} and exits 0; a crash of
the build under test shows up as a non-zero exit status.  Used by the
mutation test (each mutant must fail at least one check)."""
import json
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import test_oracle_blocks as B  # noqa: E402
import test_oracle_formats as F  # noqa: E402
import test_oracle_split_modes as S  # noqa: E402
import test_oracle_auto_scale as A  # noqa: E402
from helpers import hand_blocks, row_scaled_rows  # noqa: E402


def checks():
    yield "hand_blocks", lambda o: [B.test_hand_block(o, c) for c in hand_blocks()]
    yield "e4m3_decode", F.test_e4m3_decode_all_codes
    yield "e4m3_torch", F.test_e4m3_encode_matches_torch_cast
    yield "e4m3_brute", F.test_e4m3_encode_matches_brute_force
    yield "e2m1_codec", F.test_e2m1_codec
    yield "e2m1_brute", F.test_e2m1_encode_matches_brute_force
    yield "e8m0_rule", F.test_mxfp8_scale_rule_closed_form_all_bf16
    yield "mx_ftz", F.test_mxfp8_multiplier_ftz
    yield "bf16_decode", F.test_bf16_decode_all_codes
    yield "bf16_round", F.test_bf16_round_matches_torch_rne
    yield "mx_bound", B.test_mxfp8_error_bound_and_no_saturation
    yield "nv_props", B.test_nvfp4_block_properties
    yield "nv_sat", B.test_nvfp4_scale_saturates_at_448
    yield "swz_offsets", B.test_swizzle_worked_offsets
    yield "swz_reshape", lambda o: [B.test_swizzle_matches_reshape_formulation(o, R, C)
                                    for R, C in [(130, 8), (300, 17)]]
    yield "layouts", lambda o: [B.test_quantize_rows_independent_and_layouts_agree(o, f)
                                for f in (0, 1)]
    yield "split", B.test_split_equals_per_expert
    yield "row_hand", lambda o: [S.test_row_scaled_hand_row(o, c) for c in row_scaled_rows()]
    yield "row_scale_values", S.test_row_encode_scale_special_values
    yield "row_equal_amax", S.test_row_scaled_equal_amax_reduces_to_tensor_scaled
    yield "row_max_six", S.test_row_scaled_row_max_encodes_as_six
    yield "row_split_indep", S.test_row_scaled_rows_independent_of_split
    yield "mx_split_sizes", S.test_mxfp8_split_sizes_by_hand
    yield "mx_split", S.test_mxfp8_split_equals_per_expert
    yield "tensor_amax", A.test_tensor_amax_matches_numpy
    yield "auto_scale", A.test_auto_equals_per_tensor_with_numpy_scale
    yield "auto_shared", A.test_shared_slot_takes_the_larger_amax
    yield "auto_six", A.test_slot_amax_element_encodes_as_six
    yield "rmsnorm", lambda o: [B.test_add_rmsnorm_pins(o, sc) for sc in (1.0, 1e-3)]


def main(path):
    failed, n = [], 0
    with oracle.using(path):
        for name, fn in checks():
            n += 1
            try:
                fn(oracle)
            except Exception:  # a failed pin
                failed.append(name)
                traceback.print_exc(limit=1, file=sys.stderr)
    print(json.dumps({"checks": n, "failed": failed}), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
