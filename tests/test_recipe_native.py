"""The library's host-side allocation calls (dq_sensitivity, dq_allocate_bits)
against the allocation oracle and its pins.  CPU only: these entry points take
host memory and make no HIP call.

Source: DynaQuant page (zingnex.cn), "第一步：敏感度测量" and "第二步：比特分配"."""
from __future__ import annotations

import types

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import recipe_pins
import workload
from oracle import recipe

H = 1 << 20  # a fake address; the argument checks return before touching it


def native_module() -> types.ModuleType:
    """The library's allocation calls behind the oracle's function names, so the
    same pins run on both."""
    mod = types.ModuleType("native_recipe")

    def allocate(sens, params, levels=dq.FULL_LEVELS, budget_bits=None):
        try:
            bits, steps, loss = dq.allocate_bits(sens, params, levels, budget_bits)
        except dq.DQError as e:
            raise ValueError(str(e))
        return [int(b) for b in bits], steps, loss

    mod.allocate = allocate
    mod.sensitivity = dq.sensitivity
    return mod


@pytest.mark.parametrize("check", [
    recipe_pins.check_sensitivity, recipe_pins.check_greedy_optimal_unit_cost,
    recipe_pins.check_frontier_lagrangian, recipe_pins.check_water_level,
    recipe_pins.check_hand_cases,
])
def test_native_allocator_meets_the_pins(check):
    assert check(native_module()) == []


def stack_instance(seed: int):
    """The 448-matrix stack: parameter counts of its shapes, synthetic Hessian
    traces, and sums of squares of N(0, 0.02^2) weights (params * 0.02^2
    times a seeded spread of a few per cent)."""
    shapes = workload.stack_shapes()
    params = np.array([n * k for n, k in shapes], dtype=np.int64)
    h = workload.hessian_traces(3, len(shapes))
    rng = np.random.default_rng(seed)
    sumsq = params * 0.02 ** 2 * rng.uniform(0.95, 1.05, len(shapes))
    return h, sumsq, params


@pytest.mark.parametrize("levels", [dq.NATIVE_LEVELS, dq.FULL_LEVELS], ids=["native", "full"])
@pytest.mark.parametrize("avg_bits", [4.0, 4.5, 5.7, 6.0, 8.0, 12.5, None])
def test_stack_allocation_matches_oracle(levels, avg_bits):
    h, sumsq, params = stack_instance(1)
    s_native = dq.sensitivity(h, sumsq, params)
    s_oracle = recipe.sensitivity(h, sumsq, params)
    assert s_native.tobytes() == s_oracle.tobytes()
    budget = None if avg_bits is None else int(avg_bits * int(params.sum()))
    bits, steps, loss = dq.allocate_bits(s_native, params, levels, budget)
    obits, osteps, oloss = recipe.allocate(s_oracle, params, levels, budget)
    assert bits.tolist() == obits
    assert steps == osteps
    # predicted loss: a sum of n non-negative terms in a different order
    assert abs(loss - oloss) <= len(params) * 2.0 ** -52 * oloss
    if budget is not None:
        assert int((bits.astype(np.int64) * params).sum()) <= budget


def test_knee_budget_recipe_shape():
    """At the DynaQuant knee budget (5.7 bits per parameter on average) the
    full-mode recipe puts every matrix within a few levels of 6."""
    h, sumsq, params = stack_instance(2)
    s = dq.sensitivity(h, sumsq, params)
    bits, _, _ = dq.allocate_bits(s, params, dq.FULL_LEVELS, int(5.7 * int(params.sum())))
    avg = float((bits.astype(np.int64) * params).sum()) / float(params.sum())
    assert 5.69 <= avg <= 5.7
    assert bits.min() >= 4 and bits.max() <= 9


def test_allocation_arguments_rejected():
    f = dq.dq_allocate_bits
    s = np.array([1.0, 2.0])
    p = np.array([10, 20], dtype=np.int64)
    lv = np.array([4, 8, 16], dtype=np.int32)
    out = np.zeros(2, dtype=np.int32)
    sa, pa, la, oa = s.ctypes.data, p.ctypes.data, lv.ctypes.data, out.ctypes.data
    assert f(0, pa, 2, la, 3, -1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_NULL
    assert f(sa, pa, 2, la, 3, -1, 0, 0, 0, 0, 0, 0) == dq.DQ_ERR_NULL
    assert f(sa, pa, 2, la, 3, -1, oa, 0, 0, 4, 0, 0) == dq.DQ_ERR_NULL  # steps need arrays
    assert f(sa, pa, 0, la, 3, -1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_SHAPE
    assert f(sa, pa, 2, la, 0, -1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_BITS
    for bad in ([4, 4, 8], [8, 4], [1, 4], [4, 17]):
        b = np.array(bad, dtype=np.int32)
        assert f(sa, pa, 2, b.ctypes.data, b.size, -1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_BITS
    assert f(sa, pa, 2, la, 3, 10 * 4 + 20 * 4 - 1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_BUDGET
    for sv, pv in (([np.nan, 1.0], [10, 20]), ([-1.0, 1.0], [10, 20]), ([np.inf, 1.0], [10, 20]),
                   ([1.0, 1.0], [0, 20]), ([1.0, 1.0], [10, (1 << 40) + 1])):
        sv = np.array(sv)
        pv = np.array(pv, dtype=np.int64)
        assert f(sv.ctypes.data, pv.ctypes.data, 2, la, 3, -1, oa, 0, 0, 0, 0, 0) == dq.DQ_ERR_VALUE
    assert out.tolist() == [0, 0]  # nothing written on an error
    g = dq.dq_sensitivity
    assert g(0, H, H, 1, H) == dq.DQ_ERR_NULL
    assert g(H, H, H, 0, H) == dq.DQ_ERR_SHAPE
    for hv, sv, pv in (([np.nan], [1.0], [1]), ([1.0], [-1.0], [1]), ([1.0], [1.0], [0])):
        hv, sv, pv = np.array(hv), np.array(sv), np.array(pv, dtype=np.int64)
        assert g(hv.ctypes.data, sv.ctypes.data, pv.ctypes.data, 1, H) == dq.DQ_ERR_VALUE


def test_step_capacity_truncates_but_counts():
    s = np.array([3.0, 0.25])
    p = np.array([2, 3], dtype=np.int64)
    lv = np.array(dq.FULL_LEVELS, dtype=np.int32)
    out = np.zeros(2, dtype=np.int32)
    sm = np.full(5, -1, dtype=np.int64)
    sb = np.full(5, -1, dtype=np.int32)
    n = np.zeros(1, dtype=np.int64)
    st = dq.dq_allocate_bits(s.ctypes.data, p.ctypes.data, 2, lv.ctypes.data, lv.size, -1,
                             out.ctypes.data, sm.ctypes.data, sb.ctypes.data, 3, n.ctypes.data, 0)
    assert st == dq.DQ_OK
    assert int(n[0]) == 24 and out.tolist() == [16, 16]
    _, osteps, _ = recipe.allocate([3.0, 0.25], [2, 3], dq.FULL_LEVELS, None)
    assert list(zip(sm[:3].tolist(), sb[:3].tolist())) == osteps[:3]
    assert sm[3:].tolist() == [-1, -1] and sb[3:].tolist() == [-1, -1]
