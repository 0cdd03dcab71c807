"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs at sizes the oracle finishes quickly: several tiles and ragged tails,
every bit width, special rows and special activations.

Bars: quantize / pack / unpack bit-exact (packed words, scale bit patterns,
codes, dequantized fp32); GEMV / GEMM |y - y_ref| <= 1e-4 * sum_k |x * w_hat|
with y_ref in fp64 (exactly 0 where that sum is 0)."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, f32_bits, report, torch, u32, weights_gpu
from pins import within_tolerance

pytestmark = pytest.mark.gpu

QUANT_SHAPES = [(1, 1), (3, 31), (5, 33), (7, 255), (2, 614), (64, 256), (33, 1000), (9, 8192 + 40)]


def special_rows(K: int, bits: int) -> np.ndarray:
    """fp32 rows exercising the quantizer's corner cases."""
    qmax = (1 << (bits - 1)) - 1
    s0 = 2.0 ** -6
    rows = np.zeros((10, K), np.float32)
    idx = np.arange(K)
    rows[1] = 0.7 * np.where(idx % 2 == 0, 1, -1)  # constant magnitude, +-absmax
    lv = (idx % (2 * qmax + 1)) - qmax  # every level exactly: w = j * s0
    rows[2] = lv * s0
    ties = ((idx % 12) - 6 + 0.5) * s0  # exact (j + 1/2) * s0
    ties[0] = qmax * s0
    rows[3] = ties
    rows[4] = -0.0  # signed zeros
    rows[5] = np.where(idx % 3 == 0, 3e-39, -1e-39)  # subnormal absmax
    rows[5][0] = 5e-45
    rows[6] = 1.4e-45 * (idx % 2)  # smallest subnormal / zero
    rows[7] = np.where(idx % 2 == 0, 3.0e38, -1.0e38)  # near the top of the range
    rows[8] = np.where(idx % 5 == 0, 0.5, 2.0 ** -30)  # wide dynamic range
    rows[9] = 0.01 * (idx - K / 2) / max(K, 1)
    rows[9][K // 2] = np.nan if K > 1 else np.inf  # a non-finite row
    return rows


def run_quantize(w_np: np.ndarray, bits: int):
    report("quantize_pack shape=%s dtype=%s bits=%d" % (w_np.shape, w_np.dtype, bits))
    packed, scales = dq.quantize_pack(weights_gpu(w_np), bits)
    torch().cuda.synchronize()
    return u32(packed), f32_bits(scales)


def assert_quantize_parity(w_np: np.ndarray, bits: int):
    packed, scales = run_quantize(w_np, bits)
    o_packed, o_scales, o_q = oracle.quantize_pack(w_np, bits)
    assert np.array_equal(scales, o_scales.view(np.uint32)), "scale bits differ"
    if not np.array_equal(packed, o_packed):
        bad = np.argwhere(packed != o_packed)[:5]
        pytest.fail("packed words differ at %s" % bad.tolist())
    return o_packed, o_scales, o_q


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_pack_bitexact_bf16(bits):
    for i, (N, K) in enumerate(QUANT_SHAPES):
        w = workload.weights(11, bits * 100 + i, N, K, outlier_frac=0.01 if N * K > 100 else 0.0)
        assert_quantize_parity(w, bits)
    t5 = workload.weights(12, bits, 40, 2000, dist="t5")
    assert_quantize_parity(t5, bits)


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_pack_bitexact_f32(bits):
    for i, (N, K) in enumerate(QUANT_SHAPES):
        w = workload.weights(13, bits * 100 + i, N, K, dtype="f32")
        assert_quantize_parity(w, bits)


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_special_rows(bits):
    for K in (1, 7, 33, 64, 300, 512):
        rows = special_rows(K, bits)
        assert_quantize_parity(rows, bits)
        bf = workload.bf16_from_f32(rows)
        assert_quantize_parity(bf, bits)


@pytest.mark.parametrize("bits", range(2, 16))
def test_unpack_bitexact(bits):
    for i, (N, K) in enumerate(QUANT_SHAPES):
        w = workload.weights(14, bits * 100 + i, N, K)
        o_packed, o_scales, o_q = oracle.quantize_pack(w, bits)
        q_ref, w_ref = oracle.unpack(o_packed, o_scales, N, K, bits)
        report("unpack N=%d K=%d bits=%d" % (N, K, bits))
        P = torch().from_numpy(o_packed.view(np.int32)).cuda()
        S = torch().from_numpy(o_scales).cuda()
        q, w_hat = dq.unpack(P, S, K, bits, want_q=True, want_w=True)
        q_only, _ = dq.unpack(P, None, K, bits, want_q=True, want_w=False)
        _, w_only = dq.unpack(P, S, K, bits, want_q=False, want_w=True)
        torch().cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_ref)
        assert np.array_equal(q_only.cpu().numpy(), q_ref)
        assert np.array_equal(f32_bits(w_hat), w_ref.view(np.uint32))
        assert np.array_equal(f32_bits(w_only), w_ref.view(np.uint32))


def run_matmul(kind: str, x_np, packed_np, scales_np, K: int, bits: int):
    fn = dq.gemv if kind == "gemv" else dq.gemm
    report("%s M=%d N=%d K=%d bits=%d" % (kind, x_np.shape[0], packed_np.shape[0], K, bits))
    P = torch().from_numpy(packed_np.view(np.int32)).cuda()
    S = torch().from_numpy(scales_np).cuda()
    y = fn(bf16_gpu(x_np), P, S, K, bits)
    torch().cuda.synchronize()
    return y.cpu().numpy()


def assert_matmul_parity(kind: str, M: int, N: int, K: int, bits: int, seed: int):
    w = workload.weights(21, seed, N, K, outlier_frac=0.001)
    x = workload.activations(21, seed, M, K)
    o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
    y_ref, bound = oracle.matmul(x, o_packed, o_scales, N, K, bits)
    y = run_matmul(kind, x, o_packed, o_scales, K, bits)
    ok = within_tolerance(y, y_ref, bound)
    if not ok.all():
        m, n = np.argwhere(~ok)[0]
        pytest.fail("%s M=%d N=%d K=%d b=%d: y[%d,%d]=%r ref %r bound %r (%d bad)" % (
            kind, M, N, K, bits, m, n, y[m, n], y_ref[m, n], bound[m, n], int((~ok).sum())))


# (33, 5152) and (17, 224): K a multiple of 32 but not of 128, so the last
# 128-wide K step of the matrix-core paths is partial
GEMV_SHAPES = [(1, 1), (37, 1000), (300, 4096 + 37), (8, 17408), (40, 6144), (70, 2048),
               (33, 5152), (17, 224)]


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemv_parity(bits):
    for M in (1, 2, 3, 5, 8, 13, 16):
        for i, (N, K) in enumerate(GEMV_SHAPES):
            assert_matmul_parity("gemv", M, N, K, bits, seed=bits * 1000 + M * 10 + i)


GEMM_SHAPES = [(1, 64, 64), (7, 129, 100), (128, 128, 1000), (200, 259, 517), (257, 300, 2048)]


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemm_parity(bits):
    for i, (M, N, K) in enumerate(GEMM_SHAPES):
        assert_matmul_parity("gemm", M, N, K, bits, seed=bits * 1000 + 500 + i)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("bits", [2, 6, 9, 10, 15])
def test_one_hot_is_exact(kind, bits):
    """x = e_k picks column k of the dequantized matrix: y[k, n] = fl32(s[n] * q[n, k])."""
    N, K = 70, 16 if kind == "gemv" else 40
    w = workload.weights(22, bits, N, K)
    o_packed, o_scales, o_q = oracle.quantize_pack(w, bits)
    eye = workload.bf16_from_f32(np.eye(K, dtype=np.float32))
    y = run_matmul(kind, eye, o_packed, o_scales, K, bits)
    want = (o_scales[None, :] * o_q.T.astype(np.float32)).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_zero_rows_and_nan_scale(kind):
    bits, N, K = 6, 20, 96
    w = workload.weights(23, 0, N, K, dtype="f32")
    w[3] = 0
    w[7, 5] = np.nan
    o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
    x = workload.activations(23, 0, 4, K)
    y = run_matmul(kind, x, o_packed, o_scales, K, bits)
    assert np.all(y[:, 3] == 0)
    assert np.all(np.isnan(y[:, 7]))
    y_ref, bound = oracle.matmul(x, o_packed, o_scales, N, K, bits)
    keep = np.arange(N) != 7
    assert within_tolerance(y[:, keep], y_ref[:, keep], bound[:, keep]).all()


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_deterministic(kind):
    bits, M, N, K = 5, 3, 500, 3000
    w = workload.weights(24, 0, N, K)
    x = workload.activations(24, 0, M, K)
    o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
    y1 = run_matmul(kind, x, o_packed, o_scales, K, bits)
    y2 = run_matmul(kind, x, o_packed, o_scales, K, bits)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_quantize_then_matmul_end_to_end():
    """Whole path on the GPU: W -> dq_quantize_pack -> dq_gemv / dq_gemm, checked
    against the oracle's own quantization and fp64 product."""
    bits, M, N, K = 6, 4, 256, 256
    w = workload.weights(1, 0, N, K, dtype="f32")
    x = workload.activations(1, 0, M, K)
    report("end-to-end N=%d K=%d bits=%d" % (N, K, bits))
    P, S = dq.quantize_pack(weights_gpu(w), bits)
    X = bf16_gpu(x)
    yv = dq.gemv(X, P, S, K, bits)
    ym = dq.gemm(X, P, S, K, bits)
    torch().cuda.synchronize()
    o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
    assert np.array_equal(u32(P), o_packed)
    y_ref, bound = oracle.matmul(x, o_packed, o_scales, N, K, bits)
    assert within_tolerance(yv.cpu().numpy(), y_ref, bound).all()
    assert within_tolerance(ym.cpu().numpy(), y_ref, bound).all()


@pytest.mark.parametrize("nbytes,nparts", [(16, 1), (16, 3), (4096 + 16, 7), ((1 << 20) + 48, 2048),
                                           (12 * (1 << 20), 2048)])
def test_stream_read_reads_every_word(nbytes, nparts):
    """The streaming-read yardstick: share p of the 16-byte pieces is
    [n16 p / nparts, n16 (p + 1) / nparts) and its XOR lands in partial[p]."""
    rng = np.random.default_rng(nbytes + nparts)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    report("stream_read bytes=%d nparts=%d" % (nbytes, nparts))
    buf = torch().from_numpy(words.view(np.int32)).cuda()
    part = dq.stream_read(buf, nparts)
    torch().cuda.synchronize()
    got = part.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    pieces = words.reshape(n16, 4)
    want = np.zeros(nparts, dtype=np.uint32)
    for p in range(nparts):
        lo, hi = n16 * p // nparts, n16 * (p + 1) // nparts
        if hi > lo:
            want[p] = np.bitwise_xor.reduce(pieces[lo:hi].ravel())
    assert np.array_equal(got, want)


def test_random_shapes_whole_path():
    """Seeded random shapes, widths, dtypes and M through the whole GPU path
    (quantize + pack on the GPU, then GEMV or GEMM on its output), each checked
    in full against the oracle: bit-exact packed words and scales, products
    within 1e-4 * sum |x * w_hat|."""
    rng = np.random.default_rng(20261203)
    for case in range(40):
        bits = int(rng.integers(2, 16))
        N = int(rng.integers(1, 700))
        K = int(rng.choice([int(rng.integers(1, 3000)), 32 * int(rng.integers(1, 90)),
                            64 * int(rng.integers(1, 45))]))
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        kind = "gemv" if case % 2 == 0 else "gemm"
        M = int(rng.integers(1, 17)) if kind == "gemv" else int(rng.integers(1, 300))
        outliers = 0.001 if rng.random() < 0.3 else 0.0
        w = workload.weights(30, case, N, K, dtype=dtype, outlier_frac=outliers)
        x = workload.activations(30, case, M, K)
        report("random case %d: %s M=%d N=%d K=%d b=%d %s" % (case, kind, M, N, K, bits, dtype))
        P, S = dq.quantize_pack(weights_gpu(w), bits)
        y = (dq.gemv if kind == "gemv" else dq.gemm)(bf16_gpu(x), P, S, K, bits)
        torch().cuda.synchronize()
        o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
        assert np.array_equal(u32(P), o_packed), "case %d: packed words differ" % case
        assert np.array_equal(f32_bits(S), o_scales.view(np.uint32)), "case %d: scales differ" % case
        y_ref, bound = oracle.matmul(x, o_packed, o_scales, N, K, bits)
        ok = within_tolerance(y.cpu().numpy(), y_ref, bound)
        assert ok.all(), "case %d: %d outputs out of tolerance" % (case, int((~ok).sum()))


# K whose chunk count fills the last 64-chunk slice of a row poorly (160 and
# 65 chunks): the resident-x GEMV then takes two rows per wave; odd N leaves
# the last wave a single row (544 chunks stays at one row per wave)
TWO_ROW_SHAPES = [(37, 5120), (300, 5120), (1, 5120), (9, 17408), (33, 2080), (2, 2080)]


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemv_two_rows_per_wave(bits):
    for M in (1, 2):
        for i, (N, K) in enumerate(TWO_ROW_SHAPES):
            assert_matmul_parity("gemv", M, N, K, bits, seed=bits * 2000 + M * 10 + i)


@pytest.mark.parametrize("bits", [2, 6, 15])
def test_nonfinite_rows_counted(bits):
    """dq_quantize_pack's optional output counts the rows holding a NaN or an
    infinity (the rows whose scale is NaN), counting from zero on every call;
    the codes and scales are those of the call without it."""
    rng = np.random.default_rng(bits)
    cases = []
    for N, K in ((10, 33), (300, 4096), (7, 1), (1000, 96)):
        w = workload.weights(36, N + K, N, K, dtype="f32")
        hit = rng.random(N) < 0.2
        for n in np.flatnonzero(hit):
            w[n, rng.integers(0, K)] = rng.choice([np.nan, np.inf, -np.inf])
        cases.append(w)
    cases.append(special_rows(300, bits))
    cases.append(np.zeros((5, 64), np.float32))
    nf = torch().zeros(1, dtype=torch().int32, device="cuda")
    for w in cases:
        want = int((~np.isfinite(w)).any(axis=1).sum())
        report("nonfinite_rows shape=%s bits=%d want=%d" % (w.shape, bits, want))
        P, S = dq.quantize_pack(weights_gpu(w), bits, nonfinite=nf)
        P0, S0 = dq.quantize_pack(weights_gpu(w), bits)
        torch().cuda.synchronize()
        assert int(nf.item()) == want
        assert int(np.isnan(S.cpu().numpy()).sum()) == want
        assert np.array_equal(u32(P), u32(P0)) and np.array_equal(f32_bits(S), f32_bits(S0))
