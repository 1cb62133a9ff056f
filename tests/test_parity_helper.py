"""The comparison helper itself (CPU): one wrong row among tens of thousands
passes the whole-tensor max-abs and rel_l2 bounds, and only the per-row bound
stops it."""
import numpy as np
import pytest

from parity import MAX_ABS, REL_L2, ROW_REL_L2, assert_close, metrics


def _outputs(seed=0, rows=32768, D=64, scale=0.02):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((rows, D)) * scale  # attention-output magnitudes
    got = ref * (1 + rng.standard_normal((rows, D)) * 2e-3)  # bf16-level error
    return got, ref


def test_close_outputs_pass():
    got, ref = _outputs()
    m = assert_close(got, ref, "bf16-level error")
    assert m["row_rel_l2_max"] < ROW_REL_L2


def test_one_wrong_row_is_caught_by_the_row_bound_only():
    got, ref = _outputs()
    got[12345] = ref[12345] * 1.3  # one row 30% off
    m = metrics(got, ref)
    assert m["max_abs"] <= MAX_ABS and m["rel_l2"] <= REL_L2  # the whole-tensor bounds miss it
    assert m["row_rel_l2_max"] > 0.25
    with pytest.raises(AssertionError, match="worst row"):
        assert_close(got, ref, "one wrong row")


def test_all_zero_reference_rows_fall_back_to_the_element_bound():
    got, ref = _outputs(rows=100)
    ref[7] = 0.0
    got[7] = 1e-4  # a fully masked query: reference 0, tiny output
    assert metrics(got, ref)["row_rel_l2_max"] < ROW_REL_L2
    got[7] = 0.5
    with pytest.raises(AssertionError):
        assert_close(got, ref, "masked row")
