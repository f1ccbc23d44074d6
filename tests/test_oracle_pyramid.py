"""Pins of oracle.pyramid_budgets ([KVC] "Alocação piramidal com o PyramidKV")."""
import math

import pytest

import oracle


@pytest.mark.parametrize("n_layers,b_base,b_target", [
    (2, 64, 128), (4, 64, 128), (32, 128, 2048), (32, 0, 1000), (7, 100, 100), (5, 10, 13), (80, 512, 5275),
    (3, 9, 7),  # top budget above the target: the pyramid inverts, still exact
])
def test_budget_sum_is_the_global_target(n_layers, b_base, b_target):
    b = oracle.pyramid_budgets(n_layers, b_base, b_target)
    assert len(b) == n_layers
    assert sum(b) == n_layers * b_target
    assert all(isinstance(x, int) for x in b)


@pytest.mark.parametrize("n_layers,b_base,b_target", [(4, 64, 128), (32, 128, 2048), (9, 5, 6), (80, 512, 5275)])
def test_each_budget_is_the_linear_law_rounded_down_or_up_by_one(n_layers, b_base, b_target):
    """Against the law written with the slope solved by hand from the sum constraint,
    in floating point: B_l lies in [floor(real), floor(real) + 1], the top layer is B_base
    and the budgets do not increase with depth."""
    b = oracle.pyramid_budgets(n_layers, b_base, b_target)
    slope = (2.0 * b_target - 2.0 * b_base) / (n_layers - 1)  # dB / (N_L - 1)
    for l, x in enumerate(b):
        real = b_base + slope * (n_layers - 1 - l)
        assert math.floor(real + 1e-9) <= x <= math.floor(real + 1e-9) + 1, (l, x, real)
    assert b[-1] == b_base
    assert all(b[i] >= b[i + 1] for i in range(n_layers - 1))


def test_hand_computed_example():
    """N_L = 4, B_base = 64, B_target = 128: dB = 128, real budgets 192, 149 1/3, 106 2/3, 64;
    rounded down they sum to 511, so layer 0 gets the one lost token."""
    assert oracle.pyramid_budgets(4, 64, 128) == [193, 149, 106, 64]


def test_degenerate_cases():
    assert oracle.pyramid_budgets(1, 10, 77) == [77]
    assert oracle.pyramid_budgets(6, 50, 50) == [50] * 6          # no slope
    assert oracle.pyramid_budgets(2, 0, 3) == [6, 0]              # exact: B_0 = 2 B_target - B_base
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(3, 300, 100)                       # B_0 = -100
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(0, 1, 1)


def test_brute_force_rounding_rule_tiny():
    """Among all integer vectors within one of the real budgets, with the exact sum, the
    oracle's is the one that rounds down and gives the remainder to the lowest layers."""
    import itertools

    for n, bb, bt in [(3, 2, 5), (4, 1, 3), (5, 3, 4)]:
        real = [bb + 2 * (bt - bb) * (n - 1 - l) / (n - 1) for l in range(n)]
        cands = []
        for ups in itertools.product([0, 1], repeat=n):
            v = [math.floor(r + 1e-9) + u for r, u in zip(real, ups)]
            if sum(v) == n * bt:
                cands.append(v)
        # the lost tokens go to the lowest layers: the lexicographically largest candidate
        assert oracle.pyramid_budgets(n, bb, bt) == max(cands)
