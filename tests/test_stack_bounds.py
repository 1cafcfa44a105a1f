"""The end-to-end bounds table (golden/stack_bounds.txt) against the script that
writes it from the oracle: every whole-decoder or whole-encoder configuration the GPU tests
compare has an entry, and recomputing cheap entries gives the stored numbers."""
import os
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_stack_bounds as MSB  # noqa: E402
import stack_cases as SC  # noqa: E402


def test_every_stack_case_has_a_bound():
    table = MSB.read()
    assert set(table) == set(SC.STACK_CASES)
    for name, (bmax, bmean) in table.items():
        # max|d|/max|ref| and mean|d|/mean|ref| are normalised apart, so either
        # may be the larger
        assert 0 < bmax < 0.05 and 0 < bmean < 0.05, name


@pytest.mark.parametrize("name", ["random4", "random5", "small_t5", "enc_small"])
def test_stored_bound_is_the_scripts(name):
    drifts, _ = MSB.measure(SC.STACK_CASES[name])
    bmax, bmean = MSB.bound(drifts)
    smax, smean = MSB.read()[name]
    assert bmax == pytest.approx(smax, rel=1e-4) and bmean == pytest.approx(smean, rel=1e-4)
