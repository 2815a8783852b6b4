"""GPU parity on a seeded random sweep of small problems (the cases and how
they are drawn: tests/sweep_cases.py): every case against the fp64 oracle,
element by element, to the tolerance of its input dtype (and the derived
per-element bound for bf16 outputs)."""
import pytest

from tests.gpu_util import check_parity
from tests.sweep_cases import SWEEP_SEEDS, sweep_cases

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [w for sd in SWEEP_SEEDS for w in sweep_cases(sd)],
                         ids=lambda w: w.name)
def test_sweep_parity(wl):
    check_parity(wl, seed=7)
