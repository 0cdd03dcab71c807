"""Mutation check of the allocation pins: plant plausible mistakes in a copy of
the oracle's allocation module (loaded from text, never written to disk) and
require that the pins reject every mutant.  The committed oracle is untouched."""
from __future__ import annotations

import os
import types

import pytest

from oracle import recipe
import recipe_pins

SRC = os.path.join(os.path.dirname(recipe.__file__), "recipe.py")

# (name, text in oracle/recipe.py, replacement)
MUTANTS = [
    ("priority_not_per_byte", "return gain / nbytes", "return gain"),
    ("loss_halves_per_bit", "lo = math.ldexp(1.0, -2 * b_from)", "lo = math.ldexp(1.0, -b_from)"),
    ("top_level_lossy", "hi = 0.0 if b_to >= TOP_BITS else math.ldexp(1.0, -2 * b_to)",
     "hi = math.ldexp(1.0, -2 * b_to)"),
    ("ties_to_higher_index", "i = int(np.argmax(prio))",
     "i = int(len(prio) - 1 - np.argmax(prio[::-1]))"),
    ("stop_at_first_misfit", "prio[i] = -np.inf  # dropped: it cannot fit later either\n"
     "            continue", "break"),
    ("budget_exclusive", "if used + cost > budget:", "if used + cost >= budget:"),
    ("zero_gain_taken", "    prio[prio <= 0] = -np.inf\n", ""),
    ("start_one_level_up", "lvl = [0] * n", "lvl = [min(1, len(levels) - 1)] * n"),
    ("sensitivity_without_mean", "mean = float(ss[i]) / float(int(p[i]))", "mean = float(ss[i])"),
    ("sumsq_of_abs", "out[n] = math.fsum((row * row).tolist())",
     "out[n] = math.fsum(np.abs(row).tolist())"),
    ("sumsq_in_fp32", "row = f[n].astype(np.float64)", "row = f[n].astype(np.float32)"),
    ("nan_row_zero", "out[n] = math.nan", "out[n] = 0.0"),
]


def load_mutant(old: str, new: str) -> types.ModuleType:
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, "mutation site not found exactly once: %r" % old
    mod = types.ModuleType("recipe_mutant")
    exec(compile(text.replace(old, new), "recipe_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes():
    mod = types.ModuleType("recipe_copy")
    exec(compile(open(SRC, encoding="utf-8").read(), "recipe_copy", "exec"), mod.__dict__)
    assert recipe_pins.all_checks(mod) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_caught(name, old, new):
    mod = load_mutant(old, new)
    try:
        bad = recipe_pins.all_checks(mod)
    except Exception as e:  # a crash is a rejection too
        bad = ["raised %r" % e]
    assert bad, "mutant %s passed every pin" % name
