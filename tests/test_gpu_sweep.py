"""GPU parity on a seeded random sweep of small problems (the cases and how
they are drawn: tests/sweep_cases.py): every case against the fp64 oracle,
element by element, to the tolerance of its input dtype (and the derived
per-element bound for bf16 outputs)."""
import pytest

from tests.gpu_util import check_parity
from tests.sweep_cases import sweep_cases

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", sweep_cases(), ids=lambda w: w.name)
def test_sweep_parity(wl):
    check_parity(wl, seed=7)
