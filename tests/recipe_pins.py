"""Independent checks that pin the bit-allocation oracle (``oracle/recipe.py``)
to the mathematics and to the readings it states.  None of them re-runs the
oracle's own arithmetic: they use exact rational arithmetic (fractions),
brute-force search over every allocation, closed forms and cases worked out by
hand.

Source: DynaQuant page (zingnex.cn), "第一步：敏感度测量" (sensitivity = Hessian
trace times mean(w^2)) and "第二步：比特分配" (water-filling on a max-heap, one
bit level per step, priority = quality gained per byte; levels {4, 8, 16} or
4..16).

Each ``check_*`` takes the module under test and returns a list of violations
(empty = pass), so that the mutation tests can assert that a planted mistake
is caught.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np


def exact_loss(sens, bits) -> Fraction:
    """sum_i S_i * 4^-b_i in exact arithmetic (16 bits: no loss)."""
    tot = Fraction(0)
    for s, b in zip(sens, bits):
        if b < 16:
            tot += Fraction(s) / (4 ** b)
    return tot


def check_row_sumsq(rec) -> list[str]:
    bad = []
    # constant rows: K * c^2 exactly (bf16 0x3F00 = 0.5, 0xC040 = -3.0)
    for bits16, val in ((0x3F00, 0.5), (0xC040, -3.0)):
        for K in (1, 7, 300):
            got = rec.row_sumsq(np.full((1, K), bits16, dtype=np.uint16))[0]
            if got != K * val * val:
                bad.append("row_sumsq constant %r K=%d: %r" % (val, K, got))
    # 1, 2, ..., n (fp32): n (n + 1) (2n + 1) / 6
    for n in (1, 10, 1000):
        got = rec.row_sumsq(np.arange(1, n + 1, dtype=np.float32)[None, :])[0]
        if got != n * (n + 1) * (2 * n + 1) // 6:
            bad.append("row_sumsq 1..%d: %r" % (n, got))
    # random fp32 rows spanning many binades: the exact rational sum, rounded once
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((6, 257)) * np.exp2(rng.integers(-30, 30, (6, 257)))).astype(np.float32)
    w[1, ::3] = -w[1, ::3]
    got = rec.row_sumsq(w)
    for n in range(w.shape[0]):
        want = float(sum(Fraction(float(v)) ** 2 for v in w[n]))
        if got[n] != want:
            bad.append("row_sumsq random row %d: %r != %r" % (n, got[n], want))
    # NaN and infinity
    w = np.zeros((3, 4), dtype=np.float32)
    w[0, 1] = np.inf
    w[1, 2] = np.nan
    w[1, 0] = -np.inf
    got = rec.row_sumsq(w)
    if not (got[0] == math.inf and math.isnan(got[1]) and got[2] == 0.0):
        bad.append("row_sumsq non-finite rows: %r" % (got,))
    return bad


def check_sensitivity(rec) -> list[str]:
    bad = []
    got = rec.sensitivity([2.0, 0.5, 3.0], [8.0, 6.0, 1.0], [4, 3, 10])
    want = [2.0 * (8.0 / 4), 0.5 * (6.0 / 3), 3.0 * 0.1]
    if list(got) != want:
        bad.append("sensitivity h * sumsq / params: %r != %r" % (list(got), want))
    return bad


def brute_frontier(sens, params, levels):
    """(cost, minimum exact loss over every allocation costing at most cost),
    for every cost some allocation has, by enumerating all allocations."""
    table = sorted((sum(p * b for p, b in zip(params, bits)), exact_loss(sens, bits))
                   for bits in itertools.product(levels, repeat=len(sens)))
    out, best = [], None
    for cost, loss in table:
        best = loss if best is None or loss < best else best
        out.append((cost, best))
    return out


def brute_min_loss(frontier, budget) -> Fraction:
    best = None
    for cost, loss in frontier:
        if cost > budget:
            break
        best = loss
    return best


def check_greedy_optimal_unit_cost(rec) -> list[str]:
    """Every step of the full mode costs the same when the matrices have the
    same size, and the loss removed by successive steps of one matrix shrinks.
    For such separable problems the marginal greedy is optimal at every budget
    (the marginal-allocation theorem of Gross and of Fox): the allocator's
    loss must equal the brute-force minimum over all allocations."""
    bad = []
    levels = tuple(range(4, 17))
    rng = np.random.default_rng(11)
    for trial in range(6):
        n = 3
        sens = [float(4.0 ** rng.uniform(-2, 16)) for _ in range(n)]
        if trial == 0:
            sens = [4.0 ** 15, 3.0 * 4.0 ** 13, 4.0 ** 14]  # steps to 15 and 16 compete
        params = [5] * n
        frontier = brute_frontier(sens, params, levels)
        for budget in range(5 * 4 * n, 5 * 16 * n + 1, 5):
            bits, steps, loss = rec.allocate(sens, params, levels, budget)
            if sum(p * b for p, b in zip(params, bits)) > budget:
                bad.append("over budget")
            got = exact_loss(sens, bits)
            want = brute_min_loss(frontier, budget)
            if got > want * (1 + Fraction(1, 10 ** 12)):
                bad.append("trial %d budget %d: loss %s > optimum %s (bits %s)"
                           % (trial, budget, float(got), float(want), bits))
    return bad


def check_frontier_lagrangian(rec) -> list[str]:
    """With no budget the allocator walks the whole frontier.  Along it the loss
    removed per byte by successive steps of one matrix shrinks (in both
    modes), so every state it passes through takes all steps worth more than
    some price per byte and none worth less: it minimises loss + price * bytes,
    and such a state is optimal among all allocations that cost no more than
    it does (Everett's theorem on Lagrange multipliers), whatever the matrix
    sizes.  Checked against brute force on matrices of different sizes."""
    bad = []
    rng = np.random.default_rng(17)
    for levels in ((4, 8, 16), tuple(range(4, 17))):
        for trial in range(4):
            sens = [float(4.0 ** rng.uniform(0, 12)) for _ in range(3)]
            params = [int(v) for v in rng.integers(1, 40, 3)]
            frontier = brute_frontier(sens, params, levels)
            bits, steps, _ = rec.allocate(sens, params, levels, None)
            cur = [levels[0]] * 3
            for k, (i, b) in enumerate(steps):
                cur[i] = b
                cost = sum(p * v for p, v in zip(params, cur))
                got = exact_loss(sens, cur)
                want = brute_min_loss(frontier, cost)
                if got > want * (1 + Fraction(1, 10 ** 12)):
                    bad.append("levels %s trial %d step %d: loss %s > optimum %s at cost %d"
                               % (levels, trial, k, float(got), float(want), cost))
                    break
    return bad


def check_water_level(rec) -> list[str]:
    """Closed form of water-filling: with S_i = 4^c_i and equal sizes, the step
    b -> b+1 of matrix i is worth a constant times 4^(c_i - b), so spending
    exactly sum_i (c_i + d) bits per parameter gives b_i = c_i + d: widths
    differ by log4 of the sensitivity ratio (half a bit per factor of two).
    Valid while every c_i + d lies in [4, 15] (the step to 16 is worth
    4/3 of the pattern and is then never reached)."""
    bad = []
    rng = np.random.default_rng(5)
    for trial in range(8):
        n = int(rng.integers(2, 40))
        c = rng.integers(0, 9, n)
        d = int(rng.integers(4 - c.min(), 15 - c.max() + 1))
        P = int(rng.integers(1, 1000))
        sens = [4.0 ** int(v) for v in c]
        want = [int(v) + d for v in c]
        budget = P * sum(want)
        bits, steps, loss = rec.allocate(sens, [P] * n, tuple(range(4, 17)), budget)
        if bits != want:
            bad.append("water level trial %d: %s != %s" % (trial, bits, want))
        if loss != float(exact_loss(sens, want)):
            bad.append("water level trial %d loss %r" % (trial, loss))
    return bad


def check_hand_cases(rec) -> list[str]:
    bad = []
    F = tuple(range(4, 17))

    def expect(name, got, want):
        if got != want:
            bad.append("%s: %s != %s" % (name, got, want))

    # hardware-native levels, two matrices of P = 8 parameters, S = (4^8, 1),
    # budget 96 bits (the floor is 64).  Step 4->8 of matrix 0 removes
    # 4^8 (4^-4 - 4^-8) = 255 for 4 bytes; that of matrix 1 removes 255 / 4^8:
    # matrix 0 goes first and uses the 32 bits left.  Its step 8 -> 16 (64
    # bits) then does not fit, nor does matrix 1's 4 -> 8 (32 bits).
    bits, steps, _ = rec.allocate([4.0 ** 8, 1.0], [8, 8], (4, 8, 16), 8 * 12)
    expect("native", bits, [8, 4])
    expect("native steps", steps, [(0, 8)])
    # a step that does not fit is dropped, a smaller one still fits: matrix 0
    # (1000 params, S = 4^10) wants 4 -> 5 first but only 500 bits are left
    # above the floor; matrix 1 (10 params) takes steps up to the budget.
    bits, steps, _ = rec.allocate([4.0 ** 10, 1.0], [1000, 10], F, 1000 * 4 + 10 * 4 + 500)
    expect("drop and continue", bits, [4, 16])
    # priority is per byte, not per step: matrix 0 (100 params, S = 4) removes
    # 4x the loss of matrix 1 (10 params, S = 1) with its step 4 -> 5 but costs
    # 10x the bytes, so matrix 1 goes first; then matrix 0's step (100 bits)
    # no longer fits in the 100 bits above the floor and matrix 1 takes 10 steps.
    bits, _, _ = rec.allocate([4.0, 1.0], [100, 10], F, 100 * 4 + 10 * 4 + 100)
    expect("per byte", bits, [4, 14])
    # equal priorities: the lower index goes first
    bits, _, _ = rec.allocate([1.0, 1.0, 1.0], [7, 7, 7], F, 7 * (4 + 4 + 4) + 7)
    expect("tie to the lower index", bits, [5, 4, 4])
    # budget covers everything: every matrix reaches 16 (BF16 kept), loss 0
    bits, steps, loss = rec.allocate([3.0, 0.25], [2, 3], F, None)
    expect("everything", bits, [16, 16])
    expect("everything loss", loss, 0.0)
    expect("everything step count", len(steps), 24)
    # a matrix with S = 0 gains nothing from a step and is never raised
    bits, steps, _ = rec.allocate([0.0, 2.0], [4, 4], F, 4 * 16 * 2)
    expect("zero sensitivity", bits, [4, 16])
    # the budget is inclusive: exactly one step's worth
    bits, _, _ = rec.allocate([1.0], [9], F, 9 * 5)
    expect("exact budget", bits, [5])
    # the recorded steps replayed from the floor give the widths
    rng = np.random.default_rng(3)
    sens = [float(v) for v in rng.lognormal(0.0, 1.0, 30)]
    params = [int(v) for v in rng.integers(1, 50, 30)]
    bits, steps, _ = rec.allocate(sens, params, (4, 8, 16), sum(params) * 7)
    cur = [4] * 30
    for i, b in steps:
        cur[i] = b
    expect("replay", cur, bits)
    # an infeasible budget is refused
    try:
        rec.allocate([1.0], [10], F, 39)
        bad.append("budget below the floor accepted")
    except ValueError:
        pass
    return bad


def all_checks(rec) -> list[str]:
    return (check_row_sumsq(rec) + check_sensitivity(rec) + check_greedy_optimal_unit_cost(rec)
            + check_frontier_lagrangian(rec) + check_water_level(rec) + check_hand_cases(rec))
