"""The comparison helpers of the GPU parity tests, checked on the CPU: the
element-wise bar catches what a per-row norm lets through (one wrong output
column at d = 4096), and the near-tie check accepts only legal alternative
top-k sets."""
import numpy as np
import pytest

from gpu_util import assert_close, check_near_tie_ids, row_rel_err


def test_one_wrong_column_fails_elementwise_but_not_rownorm():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 4096))
    got = ref.copy()
    got[:, 1234] += 0.9 * np.sqrt(np.mean(ref * ref, axis=1))  # one column off by 0.9 rms
    assert row_rel_err(got, ref).max() <= 2e-2  # the row norm alone passes it
    with pytest.raises(AssertionError, match="element err"):
        assert_close(got, ref, "bf16")


def test_bf16_rounding_passes_and_zero_rows_must_be_zero():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((8, 512))
    import torch
    got = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert_close(got, ref, "bf16")
    ref[3] = 0.0
    got[3] = 0.0
    assert_close(got, ref, "bf16")
    got[3, 7] = 1e-30
    with pytest.raises(AssertionError):
        assert_close(got, ref, "bf16")
    with pytest.raises(AssertionError, match="non-finite"):
        bad = ref.copy()
        bad[0, 0] = np.nan
        assert_close(bad, ref, "bf16")


class _R:
    def __init__(self, probs):
        self.probs = np.asarray(probs, dtype=np.float64)


def test_near_tie_ids_accepts_only_legal_alternatives():
    r = _R([[0.4, 0.3, 0.3 - 1e-9, 0.0]])
    check_near_tie_ids(np.array([[0, 2]]), r, [0])      # swap at the k-boundary: legal
    with pytest.raises(AssertionError):
        check_near_tie_ids(np.array([[0, 3]]), r, [0])  # expert 3 is far below p_(k)
    with pytest.raises(AssertionError):
        check_near_tie_ids(np.array([[1, 0]]), r, [0])  # slot order against the probabilities
    with pytest.raises(AssertionError):
        check_near_tie_ids(np.array([[0, 0]]), r, [0])  # repeated id
    with pytest.raises(AssertionError):
        check_near_tie_ids(np.array([[0, 4]]), r, [0])  # id out of range
