"""The statistic behind the sensitivity on the GPU (dq_row_sumsq and the fused
dq_quantize_pack_sumsq) against the oracle, and the whole allocation flow:
measure mean(w^2) on the GPU, build sensitivities, allocate on the host,
quantize every matrix at its width, and compare every output with the
oracle's flow on the same seeded inputs.

Bars: packed words and scales bit-exact; an fp64 sum of n squares within
(n - 1) * 2^-53 of the exact sum relative to it (every square is exact in
fp64 and the terms are non-negative, so this bounds any summation order; the
tests allow n * 2^-52); recipes (integers) identical.

Source: DynaQuant page (zingnex.cn), "第一步：敏感度测量", "第二步：比特分配",
"第三步：应用配方"."""
from __future__ import annotations

import math

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import f32_bits, report, torch, u32, weights_gpu
from oracle import recipe
from test_gpu_parity import QUANT_SHAPES, special_rows

pytestmark = pytest.mark.gpu


def sums_within(got: np.ndarray, exact: np.ndarray, count: int):
    """Each fp64 sum of ``count`` exact squares within count * 2^-52 of the exact
    value; NaN where the exact value is NaN, +inf where it is +inf."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(exact))
    fin = np.isfinite(exact)
    assert np.array_equal(got[~fin & ~np.isnan(exact)], exact[~fin & ~np.isnan(exact)])
    err = np.abs(got[fin] - exact[fin])
    bound = count * 2.0 ** -52 * exact[fin]
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "sums off at rows %s: %s vs %s" % (
        bad[:5].ravel().tolist(), got[fin][bad[:5].ravel()], exact[fin][bad[:5].ravel()])


def exact_total(w_np: np.ndarray) -> float:
    f = workload.bf16_to_f32(w_np) if w_np.dtype == np.uint16 else w_np
    return math.fsum((f.astype(np.float64).ravel() ** 2).tolist())


# beside the quantizer's shapes, rows whose K is a multiple of 32 (the
# unrolled path of dq_row_sumsq) with whole and ragged rounds of loads
SUMSQ_SHAPES = QUANT_SHAPES + [(5, 5120), (6, 8192), (3, 17408), (4, 64), (13, 96)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", SUMSQ_SHAPES)
def test_row_sumsq_parity(N, K, dtype):
    w_np = workload.weights(1, 40, N, K, dtype=dtype)
    report("row_sumsq N=%d K=%d %s" % (N, K, dtype))
    row, total = dq.row_sumsq(weights_gpu(w_np))
    torch().cuda.synchronize()
    sums_within(row.cpu().numpy(), recipe.row_sumsq(w_np), K)
    sums_within(total.cpu().numpy(), [exact_total(w_np)], N * K)


@pytest.mark.parametrize("bits", [2, 6, 9, 15])
@pytest.mark.parametrize("N,K", [(3, 31), (33, 1000), (9, 8192 + 40)])
def test_fused_sumsq_matches_both(N, K, bits):
    """The fused pass gives dq_quantize_pack's words and scales bit for bit,
    and sums within the bound (it adds in another fixed order than
    dq_row_sumsq, so the last bits may differ)."""
    w_np = workload.weights(1, 41, N, K, dtype="bf16")
    w = weights_gpu(w_np)
    report("quantize_pack_sumsq N=%d K=%d bits=%d" % (N, K, bits))
    packed, scales, row, total = dq.quantize_pack_sumsq(w, bits)
    p2, s2 = dq.quantize_pack(w, bits)
    r2, t2 = dq.row_sumsq(w)
    torch().cuda.synchronize()
    o_packed, o_scales, _ = oracle.quantize_pack(w_np, bits)
    assert np.array_equal(u32(packed), o_packed)
    assert np.array_equal(f32_bits(scales), o_scales.view(np.uint32))
    assert np.array_equal(u32(packed), u32(p2)) and np.array_equal(f32_bits(scales), f32_bits(s2))
    want = recipe.row_sumsq(w_np)
    sums_within(row.cpu().numpy(), want, K)
    sums_within(r2.cpu().numpy(), want, K)
    sums_within(total.cpu().numpy(), [exact_total(w_np)], N * K)
    sums_within(t2.cpu().numpy(), [exact_total(w_np)], N * K)


@pytest.mark.parametrize("K", [1, 33, 614])
def test_sumsq_special_rows(K):
    """Signed zeros, subnormals, values near the top of the fp32 range (squares
    far beyond fp32, fine in fp64), a NaN row, an infinite row."""
    rows = special_rows(K, 6)
    inf_row = np.zeros((1, K), np.float32)
    inf_row[0, K - 1] = -np.inf
    w_np = np.concatenate([rows, inf_row])
    report("row_sumsq special K=%d" % K)
    row, total = dq.row_sumsq(weights_gpu(w_np))
    _, _, row2, _ = dq.quantize_pack_sumsq(weights_gpu(w_np), 6)
    torch().cuda.synchronize()
    want = recipe.row_sumsq(w_np)
    sums_within(row.cpu().numpy(), want, K)
    sums_within(row2.cpu().numpy(), want, K)
    t = float(total.cpu()[0])
    if np.isnan(want).any():
        assert math.isnan(t)  # a NaN row makes the total NaN
    else:
        assert t == math.inf


def test_row_sumsq_full_size_sampled():
    """28672 x 8192 bf16 (Student-t weights): 64 seeded rows against the
    oracle, and the matrix total against the exact sum of the GPU's rows."""
    w5 = workload.WORKLOADS[5]
    w_np = workload.workload_weights(w5, 0)
    report("row_sumsq 28672x8192")
    row, total = dq.row_sumsq(weights_gpu(w_np))
    torch().cuda.synchronize()
    row = row.cpu().numpy()
    rows = np.random.default_rng(9).choice(w5.N, 64, replace=False)
    sums_within(row[rows], recipe.row_sumsq(w_np[rows]), w5.K)
    sums_within(total.cpu().numpy(), [math.fsum(row.tolist())], w5.N)


@pytest.mark.parametrize("K", [5000, 5120])
def test_deterministic(K):
    w_np = workload.weights(1, 42, 301, K, dtype="bf16")
    w = weights_gpu(w_np)
    a = [dq.row_sumsq(w) for _ in range(3)]
    f = [dq.quantize_pack_sumsq(w, 6)[2:] for _ in range(2)]
    torch().cuda.synchronize()
    for r, t in a[1:]:
        assert r.cpu().numpy().tobytes() == a[0][0].cpu().numpy().tobytes()
        assert t.cpu().numpy().tobytes() == a[0][1].cpu().numpy().tobytes()
    assert f[0][0].cpu().numpy().tobytes() == f[1][0].cpu().numpy().tobytes()
    assert f[0][1].cpu().numpy().tobytes() == f[1][1].cpu().numpy().tobytes()


@pytest.mark.parametrize("levels", [dq.NATIVE_LEVELS, dq.FULL_LEVELS], ids=["native", "full"])
def test_allocation_flow_matches_oracle(levels):
    """Two layers of a small model (attention 160 x 160 four times, MLP 544 x 160
    twice and 160 x 544): mean(w^2) measured on the GPU, sensitivities with
    synthetic Hessian traces, the recipe at 5.7 bits per parameter, every
    matrix quantized at its width and multiplied by x; the oracle runs the
    same flow.  Recipes equal, packed words and scales bit-exact, GEMV within
    1e-4 * sum |x * w_hat|."""
    shapes = [(160, 160)] * 4 + [(544, 160), (544, 160), (160, 544)]
    shapes = shapes * 2
    ws = [workload.weights(3, 100 + i, n, k) for i, (n, k) in enumerate(shapes)]
    params = np.array([n * k for n, k in shapes], dtype=np.int64)
    h = workload.hessian_traces(3, len(shapes))
    budget = int(5.7 * int(params.sum()))

    report("allocation flow: row_sumsq of %d matrices" % len(ws))
    gpu_w = [weights_gpu(w) for w in ws]
    totals = [dq.row_sumsq(w)[1] for w in gpu_w]
    torch().cuda.synchronize()
    sumsq = np.array([float(t.cpu()[0]) for t in totals])
    o_sumsq = np.array([exact_total(w) for w in ws])
    sums_within(sumsq, o_sumsq, int(params.max()))
    bits, steps, _ = dq.allocate_bits(dq.sensitivity(h, sumsq, params), params, levels, budget)
    o_bits, o_steps, _ = recipe.allocate(recipe.sensitivity(h, o_sumsq, params), params, levels,
                                         budget)
    assert bits.tolist() == o_bits and steps == o_steps

    from pins import within_tolerance
    for i, (w, b) in enumerate(zip(gpu_w, bits.tolist())):
        if b >= 16:
            continue  # BF16 kept: nothing to quantize
        n, k = shapes[i]
        report("allocation flow: matrix %d %dx%d at %d bits" % (i, n, k, b))
        packed, scales = dq.quantize_pack(w, b)
        x_np = workload.activations(3, 100 + i, 1, k)
        y = dq.gemv(weights_gpu(x_np), packed, scales, k, b)
        torch().cuda.synchronize()
        o_packed, o_scales, _ = oracle.quantize_pack(ws[i], b)
        assert np.array_equal(u32(packed), o_packed)
        assert np.array_equal(f32_bits(scales), o_scales.view(np.uint32))
        y_ref, bound = oracle.matmul(x_np, o_packed, o_scales, n, k, b)
        assert within_tolerance(y.cpu().numpy(), y_ref, bound).all()
