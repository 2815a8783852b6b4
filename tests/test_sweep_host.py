"""The random sweep's cases (tests/sweep_cases.py) are drawn on the host:
check that the draw is reproducible, that every case is one the planner
accepts, and that together they reach every route."""
import pytest

from tests.sweep_cases import N_CASES, SWEEP_SEEDS, accepted, route_of, sweep_cases

ROUTES = {"fused_single_pass", "fused_persistent", "gemm_rows", "split", "conv_only"}


@pytest.mark.parametrize("seed", SWEEP_SEEDS)
def test_sweep_is_reproducible_and_accepted(seed):
    a, b = sweep_cases(seed), sweep_cases(seed)
    assert a == b and len(a) == N_CASES
    assert all(accepted(w) for w in a)


@pytest.mark.parametrize("seed", SWEEP_SEEDS)
def test_sweep_reaches_every_route(seed):
    assert {route_of(w) for w in sweep_cases(seed)} == ROUTES


def test_sweep_names_are_unique():
    names = [w.name for sd in SWEEP_SEEDS for w in sweep_cases(sd)]
    assert len(names) == len(set(names))
