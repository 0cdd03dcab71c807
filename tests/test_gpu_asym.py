"""Parity of the asymmetric (zero-point) variant with the oracle: quantize +
pack and unpack bit-exact, GEMV / GEMM within 1e-4 * sum_k |x * w_hat| of the
fp64 reference, one-hot activations exact, on rows shifted off zero,
non-negative and non-positive rows, sparse rows (one non-zero, 90 % zeros,
all zeros) with small activations at their non-zeros, and the special rows,
through every product kernel (the resident-x and sliced GEMVs, the
matrix-core GEMVs, the 128-row, wide and fallback GEMMs).

Source: "量化" tutorial (aiknowledge.cn), "量化怎么工作" (a zero point added to
the rounded quotient for distributions not centred on zero)."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, f32_bits, report, torch, u32, weights_gpu
from pins import within_tolerance
from test_gpu_parity import GEMM_SHAPES, GEMV_SHAPES, QUANT_SHAPES, special_rows

pytestmark = pytest.mark.gpu


def shifted_weights(seed: int, N: int, K: int, dtype: str = "bf16") -> np.ndarray:
    """N(0, 0.02^2) rows moved off zero by a per-row offset in [-0.04, 0.04]; every
    fifth row non-negative, every seventh non-positive."""
    w = workload.weights(31, seed, N, K, dtype="f32")
    off = np.random.default_rng(seed).uniform(-0.04, 0.04, N).astype(np.float32)
    w = w + off[:, None]
    w[::5] = np.abs(w[::5])
    w[3::7] = -np.abs(w[3::7])
    return workload.bf16_from_f32(w) if dtype == "bf16" else w.astype(np.float32)


def assert_quantize_asym(w_np: np.ndarray, bits: int):
    report("quantize_pack_asym shape=%s dtype=%s bits=%d" % (w_np.shape, w_np.dtype, bits))
    P, S, Z = dq.quantize_pack_asym(weights_gpu(w_np), bits)
    torch().cuda.synchronize()
    o_packed, o_scales, o_zeros, _ = oracle.quantize_pack_asym(w_np, bits)
    assert np.array_equal(f32_bits(S), o_scales.view(np.uint32)), "scale bits differ"
    assert np.array_equal(Z.cpu().numpy(), o_zeros), "zero points differ"
    if not np.array_equal(u32(P), o_packed):
        pytest.fail("packed words differ at %s" % np.argwhere(u32(P) != o_packed)[:5].tolist())
    return o_packed, o_scales, o_zeros


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_asym_bitexact(bits):
    for i, (N, K) in enumerate(QUANT_SHAPES):
        assert_quantize_asym(shifted_weights(bits * 100 + i, N, K, "bf16"), bits)
        assert_quantize_asym(shifted_weights(bits * 100 + 50 + i, N, K, "f32"), bits)


@pytest.mark.parametrize("bits", [2, 5, 8, 9, 15])
def test_quantize_asym_special_rows(bits):
    for K in (1, 33, 300):
        rows = special_rows(K, bits)
        extra = np.zeros((2, K), np.float32)
        extra[0, 0] = 1.4e-45  # the range over L underflows
        extra[1] = np.abs(rows[8]) + 1.0  # all positive, far from zero
        assert_quantize_asym(np.concatenate([rows, extra]), bits)


@pytest.mark.parametrize("bits", range(2, 16))
def test_unpack_asym_bitexact(bits):
    for i, (N, K) in enumerate([(3, 31), (33, 1000), (9, 8232)]):
        w = shifted_weights(bits * 10 + i, N, K)
        o_packed, o_scales, o_zeros, _ = oracle.quantize_pack_asym(w, bits)
        q_ref, w_ref = oracle.unpack_asym(o_packed, o_scales, o_zeros, N, K, bits)
        report("unpack_asym N=%d K=%d bits=%d" % (N, K, bits))
        P = torch().from_numpy(o_packed.view(np.int32)).cuda()
        q, w_hat = dq.unpack_asym(P, torch().from_numpy(o_scales).cuda(),
                                  torch().from_numpy(o_zeros).cuda(), K, bits, want_q=True,
                                  want_w=True)
        torch().cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_ref)
        assert np.array_equal(f32_bits(w_hat), w_ref.view(np.uint32))


def sparse_weights(seed: int, N: int, K: int):
    """Rows the zero point is for ("量化怎么工作": distributions not centred on
    zero, such as non-negative ReLU outputs), made sparse, by row n % 5:
    0 one positive element (z = 0, every other code 0), 1 non-negative with
    90 % zeros, 2 non-positive with 90 % zeros (z = L), 3 all zeros, 4 one
    negative element.  Returns (bf16 weights, the positions of the one-element
    rows' non-zeros)."""
    rng = np.random.default_rng(seed)
    w = np.abs(workload.bf16_to_f32(workload.weights(35, seed, N, K, dtype="bf16")))
    keep = rng.random((N, K)) < 0.1
    keep[:, 0] = True  # at least one non-zero in the 90 %-zero rows
    kind = np.arange(N) % 5
    w[kind == 1] *= keep[kind == 1]
    w[kind == 2] *= -keep[kind == 2].astype(np.float32)
    w[kind == 3] = 0.0
    pos = rng.integers(0, K, N)
    for n in np.flatnonzero((kind == 0) | (kind == 4)):
        v = w[n, pos[n]] + 0.01
        w[n] = 0.0
        w[n, pos[n]] = v if kind[n] == 0 else -v
    return workload.bf16_from_f32(w.astype(np.float32)), pos[(kind == 0) | (kind == 4)]


def small_at(x: np.ndarray, cols: np.ndarray, seed: int) -> np.ndarray:
    """x (bf16 bits) with the columns `cols` replaced by small values of either
    sign, |x| in [0.005, 0.05], while the rest stays N(0, 1): the product is
    then small next to sum_k |x_k|, which is where a fold through sum_k x loses
    it."""
    xf = workload.bf16_to_f32(x)
    rng = np.random.default_rng(seed)
    v = rng.uniform(0.005, 0.05, (x.shape[0], len(cols))) * rng.choice([-1.0, 1.0], (x.shape[0], len(cols)))
    xf[:, cols] = v.astype(np.float32)
    return workload.bf16_from_f32(xf)


def assert_asym_product(kind: str, M: int, N: int, K: int, bits: int, seed: int,
                        sparse: bool = False):
    if sparse:
        w, cols = sparse_weights(seed, N, K)
        x = small_at(workload.activations(33, seed, M, K), cols, seed)
    else:
        w = shifted_weights(seed, N, K)
        x = workload.activations(33, seed, M, K)
    o_packed, o_scales, o_zeros, _ = oracle.quantize_pack_asym(w, bits)
    y_ref, bound = oracle.matmul_asym(x, o_packed, o_scales, o_zeros, N, K, bits)
    report("%s_asym M=%d N=%d K=%d bits=%d sparse=%d" % (kind, M, N, K, bits, sparse))
    P = torch().from_numpy(o_packed.view(np.int32)).cuda()
    S = torch().from_numpy(o_scales).cuda()
    Z = torch().from_numpy(o_zeros).cuda()
    fn = dq.gemv_asym if kind == "gemv" else dq.gemm_asym
    y = fn(bf16_gpu(x), P, S, Z, K, bits)
    torch().cuda.synchronize()
    y = y.cpu().numpy()
    if sparse:  # the sparse rows really are the hard case: most codes equal z
        assert (o_zeros[1::5] == 0).all() and (o_zeros[2::5] == (1 << bits) - 1).all()
        assert (bound[:, 3::5] == 0).all()
    ok = within_tolerance(y, y_ref, bound)
    if not ok.all():
        m, n = np.argwhere(~ok)[0]
        pytest.fail("%s_asym M=%d N=%d K=%d b=%d: y[%d,%d]=%r ref %r bound %r (%d bad)" % (
            kind, M, N, K, bits, m, n, y[m, n], y_ref[m, n], bound[m, n], int((~ok).sum())))


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemv_asym_parity(bits):
    for M in (1, 2, 3, 8, 16):
        for i, (N, K) in enumerate(GEMV_SHAPES):
            assert_asym_product("gemv", M, N, K, bits, seed=bits * 1000 + M * 10 + i)


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemv_asym_sparse_rows(bits):
    """Sparse non-negative, non-positive and all-zero rows with small
    activations at the non-zero weights, through every GEMV kernel (M <= 2:
    resident-x and sliced; 3 <= M <= 16: matrix-core, codes through LDS or
    registers)."""
    for M in (1, 2, 3, 8, 16):
        for i, (N, K) in enumerate(GEMV_SHAPES + [(45, 4096)]):
            assert_asym_product("gemv", M, N, K, bits, seed=bits * 1000 + M * 10 + i + 70000,
                                sparse=True)


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemm_asym_sparse_rows(bits):
    """The sparse rows through every GEMM kernel: the LDS-staged fallback
    (K % 64 != 0), the 128-row pipelined kernel and the 256 x 256 and
    256 x 128 wide kernels."""
    shapes = GEMM_SHAPES + [(2000, 8100, 448), (300, 30000, 448)]
    for i, (M, N, K) in enumerate(shapes):
        assert_asym_product("gemm", M, N, K, bits, seed=bits * 1000 + 500 + i + 70000, sparse=True)


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemm_asym_parity(bits):
    for i, (M, N, K) in enumerate(GEMM_SHAPES):
        assert_asym_product("gemm", M, N, K, bits, seed=bits * 1000 + 500 + i)


@pytest.mark.parametrize("bits", [3, 9, 15])
def test_asym_largest_k(bits):
    """K at the library's maximum (2^22): bit-exact quantize + pack, GEMV at
    M = 1 and M = 5, GEMM, every output."""
    N, K = 3, 1 << 22
    assert_quantize_asym(shifted_weights(bits + 4000, N, K), bits)
    for kind, M in (("gemv", 1), ("gemv", 5), ("gemm", 2)):
        assert_asym_product(kind, M, N, K, bits, seed=bits * 10 + M + 4000)


@pytest.mark.parametrize("bits", [2, 6, 9, 12])
def test_gemm_asym_wide_tiles(bits):
    """Shapes that take the 256 x 256 and the 256 x 128 wide kernels."""
    for M, N, K in ((2000, 8100, 448), (300, 30000, 448)):
        assert_asym_product("gemm", M, N, K, bits, seed=bits * 7 + M)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("bits", [2, 6, 9, 10, 15])
def test_asym_one_hot_is_exact(kind, bits):
    """x = e_k: the kernels' sum is the one product 1 * (u - z), exact, so
    y[k, n] = fl32(s[n] (u - z))."""
    N, K = 70, 16 if kind == "gemv" else 40
    w = shifted_weights(bits + 900, N, K)
    o_packed, o_scales, o_zeros, _ = oracle.quantize_pack_asym(w, bits)
    _, w_hat = oracle.unpack_asym(o_packed, o_scales, o_zeros, N, K, bits)
    eye = workload.bf16_from_f32(np.eye(K, dtype=np.float32))
    P = torch().from_numpy(o_packed.view(np.int32)).cuda()
    S = torch().from_numpy(o_scales).cuda()
    Z = torch().from_numpy(o_zeros).cuda()
    report("%s_asym one-hot bits=%d" % (kind, bits))
    fn = dq.gemv_asym if kind == "gemv" else dq.gemm_asym
    for k0 in range(0, K, 16):
        xs = eye[k0:k0 + 16]
        y = fn(bf16_gpu(xs), P, S, Z, K, bits)
        torch().cuda.synchronize()
        assert np.array_equal(f32_bits(y), w_hat.T[k0:k0 + 16].copy().view(np.uint32))


def test_quantize_asym_then_products_end_to_end():
    """GPU quantize -> GPU GEMV and GEMM, against the oracle's flow."""
    N, K, bits = 640, 2048, 5
    w = shifted_weights(4242, N, K)
    P, S, Z = dq.quantize_pack_asym(weights_gpu(w), bits)
    x = workload.activations(34, 1, 300, K)
    X = bf16_gpu(x)
    yv = dq.gemv_asym(X[:4], P, S, Z, K, bits)
    yg = dq.gemm_asym(X, P, S, Z, K, bits)
    torch().cuda.synchronize()
    o_packed, o_scales, o_zeros, _ = oracle.quantize_pack_asym(w, bits)
    y_ref, bound = oracle.matmul_asym(x, o_packed, o_scales, o_zeros, N, K, bits)
    assert within_tolerance(yv.cpu().numpy(), y_ref[:4], bound[:4]).all()
    assert within_tolerance(yg.cpu().numpy(), y_ref, bound).all()
