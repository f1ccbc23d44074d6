"""PyramidKV per-layer cache budgets (test infrastructure only).

[KVC] "Alocação piramidal com o PyramidKV": the budget of layer l falls linearly with
depth,

    B_l = B_base + dB * (N_L - 1 - l) / (N_L - 1),

B_base being the budget of the top layer, and the budgets together meet the global
target, sum_l B_l = N_L * B_target.  Since sum_l (N_L - 1 - l) / (N_L - 1) = N_L / 2,
the target fixes the slope: dB = 2 * (B_target - B_base).

The page gives real-valued budgets; a cache holds whole tokens.  Reading taken here:
each B_l is rounded down, and the tokens that rounding lost (fewer than N_L) go one
each to the lowest layers 0, 1, ..., so the sum is exact and the lower layers, which
the page says need the more detailed context, keep the extra.  One layer: B_0 = B_target.
"""
from fractions import Fraction


def pyramid_budgets(n_layers, b_base, b_target):
    """Integer budgets [B_0, ..., B_{N_L-1}] (layer 0 lowest).  Exact rational arithmetic."""
    if n_layers < 1:
        raise ValueError("n_layers must be >= 1")
    if n_layers == 1:
        return [int(b_target)]
    d_b = 2 * (Fraction(b_target) - Fraction(b_base))
    real = [Fraction(b_base) + d_b * Fraction(n_layers - 1 - l, n_layers - 1) for l in range(n_layers)]
    out = [r.numerator // r.denominator for r in real]  # floor
    lost = n_layers * b_target - sum(out)
    for l in range(lost):
        out[l] += 1
    if min(out) < 0:
        raise ValueError("a layer budget would be negative")
    return out
