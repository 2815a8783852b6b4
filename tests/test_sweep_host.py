"""The random sweep's cases (tests/sweep_cases.py) are drawn on the host:
check that the draw is reproducible, that every case is one the planner
accepts, and that together they reach every route."""
from tests.sweep_cases import N_CASES, accepted, route_of, sweep_cases

ROUTES = {"fused_single_pass", "fused_persistent", "gemm_rows", "split", "conv_only"}


def test_sweep_is_reproducible_and_accepted():
    a, b = sweep_cases(), sweep_cases()
    assert a == b and len(a) == N_CASES
    assert all(accepted(w) for w in a)


def test_sweep_reaches_every_route():
    assert {route_of(w) for w in sweep_cases()} == ROUTES
