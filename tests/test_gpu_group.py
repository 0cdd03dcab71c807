"""Parity of the group-wise scales with the oracle: quantize + pack and unpack
bit-exact, GEMV / GEMM within 1e-4 * sum_k |x * w_hat| of the fp64 reference
(here w_hat = q * s[n, k / g]), one-hot activations exact; group sizes from
one chunk to 2048, ragged last groups, K shorter than a group, groups of very
different magnitude, zero and non-finite groups.

Source: "量化" tutorial (aiknowledge.cn), exercise 1 of its exercises
section (one scale per group of weights, sizes 32 to 256)."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, f32_bits, report, torch, u32, weights_gpu
from pins import within_tolerance

pytestmark = pytest.mark.gpu

GROUPS = [32, 64, 128, 256, 2048]
SHAPES = [(1, 1), (3, 31), (5, 33), (7, 300), (33, 1000), (9, 8192 + 40), (64, 4096)]


def group_weights(seed: int, N: int, K: int, g: int, dtype: str = "bf16") -> np.ndarray:
    """N(0, 0.02^2) with every third group scaled by 30, a zero group and a
    group holding an infinity when the matrix has room for them."""
    w = workload.weights(51, seed, N, K, dtype="f32", outlier_frac=0.01 if N * K > 100 else 0.0)
    G = -(-K // g)
    for j in range(0, G, 3):
        w[:, j * g:(j + 1) * g] *= 30
    if N > 2 and G > 1:
        w[1, g:2 * g] = 0
        w[2, min(K - 1, g + 3)] = np.inf
    return workload.bf16_from_f32(w) if dtype == "bf16" else w


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_group_bitexact(bits):
    for g in GROUPS:
        for i, (N, K) in enumerate(SHAPES):
            for dtype in ("bf16", "f32"):
                w = group_weights(bits * 100 + i, N, K, g, dtype)
                report("quantize_pack_group N=%d K=%d g=%d %s b=%d" % (N, K, g, dtype, bits))
                P, S = dq.quantize_pack_group(weights_gpu(w), bits, g)
                torch().cuda.synchronize()
                o_packed, o_scales, _ = oracle.quantize_pack_group(w, bits, g)
                assert np.array_equal(f32_bits(S), o_scales.view(np.uint32)), (g, N, K, dtype)
                assert np.array_equal(u32(P), o_packed), (g, N, K, dtype)


@pytest.mark.parametrize("bits", [2, 5, 8, 11, 15])
def test_unpack_group_bitexact(bits):
    for g in (32, 128, 2048):
        N, K = 9, 1000
        w = group_weights(bits + g, N, K, g)
        o_packed, o_scales, o_q = oracle.quantize_pack_group(w, bits, g)
        q_ref, w_ref = oracle.unpack_group(o_packed, o_scales, N, K, bits, g)
        report("unpack_group g=%d b=%d" % (g, bits))
        q, w_hat = dq.unpack_group(torch().from_numpy(o_packed.view(np.int32)).cuda(),
                                   torch().from_numpy(o_scales).cuda(), K, bits, g,
                                   want_q=True, want_w=True)
        torch().cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_ref)
        assert np.array_equal(f32_bits(w_hat), w_ref.view(np.uint32))


def assert_group_product(kind, M, N, K, bits, g, seed):
    w = group_weights(seed, N, K, g)
    if N > 2:
        w[2] = workload.bf16_from_f32(np.full(K, 0.01, np.float32))  # no infinity in products
    x = workload.activations(52, seed, M, K)
    o_packed, o_scales, _ = oracle.quantize_pack_group(w, bits, g)
    y_ref, bound = oracle.matmul_group(x, o_packed, o_scales, N, K, bits, g)
    report("%s_group M=%d N=%d K=%d g=%d b=%d" % (kind, M, N, K, g, bits))
    fn = dq.gemv_group if kind == "gemv" else dq.gemm_group
    y = fn(bf16_gpu(x), torch().from_numpy(o_packed.view(np.int32)).cuda(),
           torch().from_numpy(o_scales).cuda(), K, bits, g)
    torch().cuda.synchronize()
    y = y.cpu().numpy()
    ok = within_tolerance(y, y_ref, bound)
    if not ok.all():
        m, n = np.argwhere(~ok)[0]
        pytest.fail("%s_group M=%d N=%d K=%d g=%d b=%d: y[%d,%d]=%r ref %r bound %r" % (
            kind, M, N, K, g, bits, m, n, y[m, n], y_ref[m, n], bound[m, n]))


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemv_group_parity(bits):
    for g in (32, 128, 256):
        for M in (1, 2, 5, 16):
            for i, (N, K) in enumerate([(37, 1000), (70, 2048), (8, 4096 + 37), (300, 96)]):
                assert_group_product("gemv", M, N, K, bits, g, bits * 1000 + M * 10 + i + g)


@pytest.mark.parametrize("bits", [2, 4, 7, 9, 10, 13, 15])
def test_gemv_group_matrix_core_tiles(bits):
    """3 <= M <= 16 with groups of whole 128-code steps: the matrix-core GEMV
    with 32-row tiles (N * K > 2^24), a ragged last tile, a last step of half
    its codes, and groups of one, two and four steps."""
    for M, N, K, g in ((3, 4100, 4224, 128), (9, 4100, 4160, 256), (16, 4100, 4160, 512)):
        assert_group_product("gemv", M, N, K, bits, g, bits * 100 + M)


@pytest.mark.parametrize("bits", [3, 9, 15])
def test_group_largest_k(bits):
    """K at the library's maximum (2^22) with the largest and a mid group size:
    bit-exact quantize + pack, GEMV at M = 1 (VALU kernel, x too large for LDS)
    and M = 5 (matrix-core kernel with the per-step fold), GEMM, every output."""
    N, K = 3, 1 << 22
    for g in (2048, 256):
        w = group_weights(bits + g, N, K, g)
        report("quantize_pack_group largest K g=%d b=%d" % (g, bits))
        P, S = dq.quantize_pack_group(weights_gpu(w), bits, g)
        torch().cuda.synchronize()
        o_packed, o_scales, _ = oracle.quantize_pack_group(w, bits, g)
        assert np.array_equal(f32_bits(S), o_scales.view(np.uint32))
        assert np.array_equal(u32(P), o_packed)
        for kind, M in (("gemv", 1), ("gemv", 5), ("gemm", 2)):
            assert_group_product(kind, M, N, K, bits, g, bits * 10 + M + g)


@pytest.mark.parametrize("bits", range(2, 16))
def test_gemm_group_parity(bits):
    # K = 320: five 64-code steps, so the pipelined kernel's last step runs
    # after its two-step loop and g = 128, 2048 end in a partial group
    for g in (32, 64, 128, 2048):
        for i, (M, N, K) in enumerate([(1, 64, 64), (7, 129, 100), (200, 259, 517),
                                       (257, 300, 2048), (130, 200, 320)]):
            assert_group_product("gemm", M, N, K, bits, g, bits * 1000 + 500 + i + g)


@pytest.mark.parametrize("bits", [2, 6, 9, 10, 15])
def test_gemm_group_prefill_shapes(bits):
    """Prefill-sized group-wise GEMMs (M = 256 .. 512, N up to 32768): the
    pipelined 128-row kernel with the group fold over hundreds of tiles
    (groups of one, two, eight and sixteen 64-code steps; ragged last row and
    column tiles), sampled weight rows (first and last included) against the
    oracle, every m."""
    t = torch()
    for i, (M, N, K, g) in enumerate(((512, 16384, 1024, 64), (300, 16300, 1024, 128),
                                      (256, 32768, 512, 512), (512, 16384, 1024, 1024))):
        seed = bits * 100 + 70 + i
        w = group_weights(seed, N, K, g)
        w[2] = workload.bf16_from_f32(np.full(K, 0.01, np.float32))  # no infinity in products
        x = workload.activations(52, seed, M, K)
        o_packed, o_scales, _ = oracle.quantize_pack_group(w, bits, g)
        report("gemm_group prefill M=%d N=%d K=%d g=%d b=%d" % (M, N, K, g, bits))
        y = dq.gemm_group(bf16_gpu(x), t.from_numpy(o_packed.view(np.int32)).cuda(),
                          t.from_numpy(o_scales).cuda(), K, bits, g)
        t.cuda.synchronize()
        rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(N, 62, replace=False),
                                         [0, 1, 2, N - 1]]))
        y_ref, bound = oracle.matmul_group(x, np.ascontiguousarray(o_packed[rows]),
                                           np.ascontiguousarray(o_scales[rows]), len(rows), K, bits, g)
        got = y.cpu().numpy()[:, rows]
        ok = within_tolerance(got, y_ref, bound)
        if not ok.all():
            m, j = np.argwhere(~ok)[0]
            pytest.fail("gemm_group prefill M=%d N=%d K=%d g=%d b=%d: y[%d,%d]=%r ref %r bound %r" % (
                M, N, K, g, bits, m, rows[j], got[m, j], y_ref[m, j], bound[m, j]))


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("bits", [2, 6, 9, 10, 15])
def test_group_one_hot_is_exact(kind, bits):
    """x = e_k: the group's partial sum is q[n, k] exactly and it is scaled
    once, so y[k, n] = fl32(q[n, k] * s[n, k / g])."""
    for N, K, g in ((70, 96, 32), (70, 384, 128)):  # g = 128: the matrix-core GEMV
        w = group_weights(bits + 77, N, K, g)
        w[2] = w[0]
        o_packed, o_scales, _ = oracle.quantize_pack_group(w, bits, g)
        _, w_hat = oracle.unpack_group(o_packed, o_scales, N, K, bits, g)
        eye = workload.bf16_from_f32(np.eye(K, dtype=np.float32))
        P = torch().from_numpy(o_packed.view(np.int32)).cuda()
        S = torch().from_numpy(o_scales).cuda()
        fn = dq.gemv_group if kind == "gemv" else dq.gemm_group
        report("%s_group one-hot b=%d g=%d" % (kind, bits, g))
        for k0 in range(0, K, 16):
            y = fn(bf16_gpu(eye[k0:k0 + 16]), P, S, K, bits, g)
            torch().cuda.synchronize()
            assert np.array_equal(f32_bits(y), w_hat.T[k0:k0 + 16].copy().view(np.uint32))
