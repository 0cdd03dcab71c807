"""The bit-allocation oracle against its pins (CPU only)."""
from __future__ import annotations

import pytest

from oracle import recipe
import recipe_pins


@pytest.mark.parametrize("check", [
    recipe_pins.check_row_sumsq, recipe_pins.check_sensitivity,
    recipe_pins.check_greedy_optimal_unit_cost, recipe_pins.check_frontier_lagrangian,
    recipe_pins.check_water_level,
    recipe_pins.check_hand_cases,
])
def test_recipe_oracle_pinned(check):
    assert check(recipe) == []


def test_modes_and_levels():
    assert recipe.NATIVE_LEVELS == (4, 8, 16)
    assert recipe.FULL_LEVELS == tuple(range(4, 17))
    with pytest.raises(ValueError):
        recipe.allocate([1.0], [1], (4, 4, 8), 100)
    with pytest.raises(ValueError):
        recipe.allocate([1.0], [1], (1, 4), 100)
    with pytest.raises(ValueError):
        recipe.allocate([-1.0], [1], (4, 8), 100)
    with pytest.raises(ValueError):
        recipe.allocate([1.0], [0], (4, 8), 100)
