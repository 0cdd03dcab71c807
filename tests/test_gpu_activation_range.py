"""Activations at the ends of the bf16 range, through every product kernel:
all-subnormal x (every nonzero x below 2^-126, so each product is a tiny
exact fp32 number that a flush to zero would lose entirely), x mixing
subnormal and normal magnitudes, and x near 2^100 (products far above 1 that
still fit fp32).  The tolerance is the scope's own: |y - y_ref| <= 1e-4 *
sum_k |x * w_hat| with y_ref in fp64 (y exactly 0 where the sum is 0), so a
kernel that dropped the subnormal products would fail the first case by the
whole result."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, report, torch
from pins import within_tolerance

pytestmark = pytest.mark.gpu


def activations(kind: str, seed: int, M: int, K: int) -> np.ndarray:
    """bf16 bit patterns [M, K] of the named range."""
    rng = np.random.default_rng([31, seed, M, K])
    sign = rng.integers(0, 2, (M, K)).astype(np.uint16) << 15
    mant = rng.integers(0, 128, (M, K)).astype(np.uint16)
    if kind == "subnormal":  # exponent field 0: m * 2^-133, m in 1 .. 127
        return sign | np.maximum(mant, 1)
    if kind == "mixed":  # exponents 1 .. 254 drawn so that half the entries lie below 2^-100
        e = np.where(rng.random((M, K)) < 0.5, rng.integers(1, 27, (M, K)),
                     rng.integers(100, 140, (M, K))).astype(np.uint16)
        return sign | (e << 7) | mant
    if kind == "large":  # around 2^100
        e = rng.integers(127 + 96, 127 + 104, (M, K)).astype(np.uint16)
        return sign | (e << 7) | mant
    raise ValueError(kind)


def check(y: np.ndarray, x: np.ndarray, o_packed, o_scales, N: int, K: int, bits: int, tag: str):
    y_ref, bound = oracle.matmul(x, o_packed, o_scales, N, K, bits)
    ok = within_tolerance(y, y_ref, bound)
    if not ok.all():
        m, n = np.argwhere(~ok)[0]
        pytest.fail("%s: y[%d,%d]=%r ref %r bound %r (%d bad)" % (
            tag, m, n, y[m, n], y_ref[m, n], bound[m, n], int((~ok).sum())))


# (M, N, K): resident-x GEMV (M <= 2), matrix-core GEMV (3 <= M <= 16),
# GEMM tiles with ragged edges
GEMV_CASES = [(1, 96, 4096), (2, 70, 1000), (8, 64, 2048), (16, 40, 4096 + 64)]
GEMM_CASES = [(64, 96, 1024), (300, 260, 512)]


@pytest.mark.parametrize("kind", ["subnormal", "mixed", "large"])
@pytest.mark.parametrize("bits", [4, 6, 8, 12])
def test_products_over_activation_range(kind, bits):
    for i, (M, N, K) in enumerate(GEMV_CASES + GEMM_CASES):
        fn = dq.gemv if i < len(GEMV_CASES) else dq.gemm
        w = workload.weights(32, bits * 10 + i, N, K)
        x = activations(kind, bits * 10 + i, M, K)
        o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
        tag = "%s %s M=%d N=%d K=%d bits=%d" % (fn.__name__, kind, M, N, K, bits)
        report(tag)
        P = torch().from_numpy(o_packed.view(np.int32)).cuda()
        S = torch().from_numpy(o_scales).cuda()
        y = fn(bf16_gpu(x), P, S, K, bits)
        torch().cuda.synchronize()
        check(y.cpu().numpy(), x, o_packed, o_scales, N, K, bits, tag)


@pytest.mark.parametrize("kind", ["subnormal", "mixed", "large"])
def test_batched_over_activation_range(kind):
    """The batched decode launch (row-sliced and resident-x bodies) on the same ranges."""
    items, refs = [], []
    for i, (N, K, bits) in enumerate([(64, 4096, 6), (48, 5120, 5), (40, 1000, 8), (30, 2048, 4)]):
        w = workload.weights(33, i, N, K)
        x = activations(kind, 100 + i, 1, K)
        o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
        P = torch().from_numpy(o_packed.view(np.int32)).cuda()
        S = torch().from_numpy(o_scales).cuda()
        items.append((bf16_gpu(x), P, S, K, bits))
        refs.append((x, o_packed, o_scales, N, K, bits))
    report("gemv_batched %s" % kind)
    ys = dq.gemv_batched(items)
    torch().cuda.synchronize()
    for y, (x, o_packed, o_scales, N, K, bits) in zip(ys, refs):
        check(y.cpu().numpy(), x, o_packed, o_scales, N, K, bits, "batched %s b=%d" % (kind, bits))
