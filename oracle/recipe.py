"""CPU oracle for the bit-allocation step that comes before quantization: the
per-matrix statistic mean(w^2), the sensitivity built from it, and the
water-filling allocator that turns sensitivities into a recipe (one bit width
per weight matrix).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
package never imports it and shares no code with it.

Source: DynaQuant page (zingnex.cn), sections "第一步：敏感度测量" (the
sensitivity of a matrix is its Hessian trace times the mean of its squared
weights), "第二步：比特分配" (water-filling on a max-heap: each step raises one
matrix by one bit level, the matrix whose next level buys the most quality per
byte; a hardware-native mode with levels {4, 8, 16} and a full mode with every
width from 4 to 16, 16 meaning the BF16 weights are kept) and "第三步：应用配方"
(the recipe is applied per matrix).

Readings where the page is silent (each one a plain choice):

* predicted loss of a matrix at b bits: L(b) = S * 4^-b, and L(16) = 0.  The
  sensitivity multiplies the mean squared weight by the Hessian trace; uniform
  b-bit rounding leaves an error whose power is that mean square times a
  constant times 4^-b, so S * 4^-b is the second-order loss up to a constant
  that is the same for every matrix (it cannot change the ranking).  At 16
  bits the BF16 weights are kept, which is the baseline itself: no loss;
* cost of a matrix at b bits: params * b bits (the packed payload, no row
  padding); the budget is a total number of bits;
* start: every matrix at the lowest level.  A step raises one matrix to its
  next level; its priority is the loss it removes divided by the bytes it
  adds.  The step with the highest priority goes first; equal priorities go
  to the lower matrix index;
* a step that no longer fits in the budget is dropped, and that matrix stays
  where it is (the budget only shrinks, so it can never fit later); the
  others keep going until no step is left (water is poured until nothing more
  fits);
* a step that removes no loss (S = 0) is never taken.

Arithmetic is fp64, in the order the functions below spell out, so that an
implementation doing the same operations gets the same bits.
"""
from __future__ import annotations

import math

import numpy as np

TOP_BITS = 16  # the BF16 weights kept as they are
NATIVE_LEVELS = (4, 8, 16)
FULL_LEVELS = tuple(range(4, 17))


def row_sumsq(w: np.ndarray) -> np.ndarray:
    """Sum over k of w[n, k]^2 for every row, in fp64, correctly rounded.

    ``w`` is float32, or uint16 holding bf16 bit patterns.  Every square of an
    fp32 (or bf16) value is exact in fp64, and ``math.fsum`` returns the
    correctly rounded sum of the exact squares.  A row with a NaN gives NaN; a
    row with an infinity (and no NaN) gives +inf."""
    w = np.ascontiguousarray(w)
    if w.dtype == np.uint16:
        f = (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif w.dtype == np.float32:
        f = w
    else:
        raise TypeError("w must be float32 or uint16 (bf16 bits)")
    out = np.empty(f.shape[0], dtype=np.float64)
    for n in range(f.shape[0]):
        row = f[n].astype(np.float64)
        if np.isnan(row).any():
            out[n] = math.nan
        elif np.isinf(row).any():
            out[n] = math.inf
        else:
            out[n] = math.fsum((row * row).tolist())
    return out


def matrix_sumsq(w: np.ndarray) -> float:
    """Sum of w^2 over the whole matrix, correctly rounded (fp64)."""
    return math.fsum(row_sumsq(w).tolist())


def sensitivity(h_trace, sumsq, params) -> np.ndarray:
    """S = h_trace * mean(w^2), with mean(w^2) = sumsq / params: one fp64
    divide, then one fp64 multiply, per matrix."""
    h = np.asarray(h_trace, dtype=np.float64)
    ss = np.asarray(sumsq, dtype=np.float64)
    p = np.asarray(params, dtype=np.int64)
    out = np.empty(h.shape, dtype=np.float64)
    for i in range(h.size):
        mean = float(ss[i]) / float(int(p[i]))
        out[i] = float(h[i]) * mean
    return out


def level_loss(s: float, bits: int) -> float:
    """Predicted loss of a matrix of sensitivity s kept at ``bits`` bits."""
    return 0.0 if bits >= TOP_BITS else s * math.ldexp(1.0, -2 * bits)


def step_priority(s: float, params: int, b_from: int, b_to: int) -> float:
    """Loss removed per byte added by raising a matrix from b_from to b_to bits.

    gain = s * (4^-b_from - 4^-b_to) (the difference of two powers of two is
    exact; 4^-16 is taken as 0), bytes = params * (b_to - b_from) / 8."""
    lo = math.ldexp(1.0, -2 * b_from)
    hi = 0.0 if b_to >= TOP_BITS else math.ldexp(1.0, -2 * b_to)
    gain = s * (lo - hi)
    nbytes = float(params * (b_to - b_from)) / 8.0
    return gain / nbytes


def check_inputs(sens, params, levels, budget_bits):
    sens = [float(v) for v in sens]
    params = [int(v) for v in params]
    levels = [int(v) for v in levels]
    if not sens or len(sens) != len(params):
        raise ValueError("need one sensitivity and one parameter count per matrix")
    if not levels or any(b < 2 or b > TOP_BITS for b in levels) or any(
            a >= b for a, b in zip(levels, levels[1:])):
        raise ValueError("levels must be strictly increasing widths in [2, 16]")
    if any(not math.isfinite(s) or s < 0 for s in sens):
        raise ValueError("sensitivities must be finite and >= 0")
    if any(p < 1 for p in params):
        raise ValueError("parameter counts must be >= 1")
    if int(budget_bits) < sum(p * levels[0] for p in params):
        raise ValueError("budget below every matrix at the lowest level")
    return sens, params, levels, int(budget_bits)


def allocate(sens, params, levels=FULL_LEVELS, budget_bits=None):
    """Water-filling bit allocation.

    Returns (bits, steps, loss): the width chosen for every matrix, the steps
    taken in order as (matrix, new width), and the predicted total loss
    sum_i L_i(bits_i) (correctly rounded).  ``budget_bits`` None means no
    budget: the whole frontier from the lowest to the highest levels."""
    if budget_bits is None:
        budget_bits = sum(int(p) for p in params) * int(levels[-1])
    sens, params, levels, budget = check_inputs(sens, params, levels, budget_bits)
    n = len(sens)
    lvl = [0] * n  # index into levels of every matrix's current width
    used = sum(p * levels[0] for p in params)
    # priority of every matrix's next step; -inf marks a matrix with no step left
    prio = np.full(n, -np.inf)
    for i in range(n):
        if len(levels) > 1:
            prio[i] = step_priority(sens[i], params[i], levels[0], levels[1])
    prio[prio <= 0] = -np.inf
    steps = []
    while True:
        i = int(np.argmax(prio))  # the first index among equal maxima
        if prio[i] == -np.inf:
            break
        cost = params[i] * (levels[lvl[i] + 1] - levels[lvl[i]])
        if used + cost > budget:
            prio[i] = -np.inf  # dropped: it cannot fit later either
            continue
        used += cost
        lvl[i] += 1
        steps.append((i, levels[lvl[i]]))
        if lvl[i] + 1 < len(levels):
            p = step_priority(sens[i], params[i], levels[lvl[i]], levels[lvl[i] + 1])
            prio[i] = p if p > 0 else -np.inf
        else:
            prio[i] = -np.inf
    bits = [levels[j] for j in lvl]
    loss = math.fsum(level_loss(s, b) for s, b in zip(sens, bits))
    return bits, steps, loss
