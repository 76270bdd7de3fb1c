"""CPU test of the build's assembly check for the block-scaled matrix
instruction: a destination that overlaps the A or B source is rejected."""

import pytest

from ternary_weights_hadamard_amd.build import check_scaled_mfma_operands

OK = """
\tv_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[70:77], v[50:53], 0, v39, v40 op_sel_hi:[0,0,0] blgp:4
\tv_mfma_scale_f32_16x16x128_f8f6f4 v[18:21], v[2:9], v[14:17], v[10:13], v25, v24 op_sel_hi:[0,0,0] blgp:4
\tv_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:11], v[12:15], v[0:3], v1, v1 ; in place accumulate
"""


def test_disjoint_and_in_place_forms_pass():
    assert check_scaled_mfma_operands(OK, "ok") == 3


@pytest.mark.parametrize("line", [
    "v_mfma_scale_f32_16x16x128_f8f6f4 v[2:5], v[2:9], v[14:17], v[10:13], v21, v20 op_sel_hi:[0,0,0] blgp:4",
    "v_mfma_scale_f32_16x16x128_f8f6f4 v[8:11], v[0:7], v[10:13], 0, v1, v1 blgp:4",
    "v_mfma_scale_f32_16x16x128_f8f6f4 v[2:5], v[10:17], v[2:5], v[18:21], v25, v24 blgp:4",
])
def test_overlapping_destination_is_rejected(line):
    with pytest.raises(RuntimeError):
        check_scaled_mfma_operands("\t" + line + "\n", "bad")
