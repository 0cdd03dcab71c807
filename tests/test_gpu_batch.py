"""Parity of the batched decode product (dq_gemv_batched): several matrices
of mixed widths and shapes in one call, each output within 1e-4 * sum_k
|x * w_hat| of the oracle's fp64 product.  Items on the one-row-per-wave path
(rows under 64 chunks), items at 3 <= M <= 16 (the matrix-core body of
dq_gemv, one launch for all items with K a multiple of 32) and items outside
the single launch (K not a multiple of 32, x too large for LDS) are
bit-identical to dq_gemv; streamed
items (rows of 64 chunks or more) add each chunk's sum into the row total,
so they are checked against the oracle and for the same bits on every call.
Covered: every width, rows that end inside a slice (65, 160, 544 chunks per
row), rows per wave from 1 up, ragged last workgroups and waves without rows,
the largest batch, shared activations, and the decode and layer shapes of
the workloads (sampled rows against the oracle).

Source: DynaQuant page (zingnex.cn), "自定义内核架构" (the packed codes'
bandwidth saving becomes decode speed); BPDQ article, section 3.2 (the fused
dequantizing product)."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, f32_bits, report, torch, u32, weights_gpu
from pins import within_tolerance

pytestmark = pytest.mark.gpu

# (N, K, bits): every width, K multiples of 32 (one launch) and not (own
# launch), one-row and two-rows-per-wave shapes, a ragged last workgroup
MIXED = [(300, 4096, 4), (37, 1000, 5), (70, 2048, 15), (1, 32, 2), (40, 6144, 6),
         (33, 5152, 9), (8, 17408, 7), (5, 5120, 3), (129, 2080, 8), (17, 224, 10),
         (2, 96, 11), (9, 4096 + 37, 12), (64, 256, 13), (3, 8192, 14)]


def quantized(seed, N, K, bits):
    """Packed codes and scales by the oracle (CPU), uploaded: (packed, scales)
    on the GPU and the same arrays on the host."""
    w = workload.weights(61, seed, N, K, dtype="bf16")
    o_packed, o_scales, _ = oracle.quantize_pack(w, bits)
    t = torch()
    P = t.from_numpy(o_packed.view(np.int32)).cuda()
    S = t.from_numpy(o_scales).cuda()
    return P, S, o_packed, o_scales


def oracle_rows(w_rows, rows, P, S, bits):
    """The oracle's packed codes and scales of the sampled rows (w_rows: their
    bf16 bits), which must equal the GPU's rows of P and S."""
    o_packed, o_scales, _ = oracle.quantize_pack(np.ascontiguousarray(w_rows), bits)
    idx = torch().from_numpy(np.asarray(rows)).cuda()
    assert np.array_equal(u32(P.index_select(0, idx)), o_packed), "packed rows differ"
    assert np.array_equal(f32_bits(S.index_select(0, idx)), o_scales.view(np.uint32))
    return o_packed, o_scales


def streamed(M, K):
    return M <= 2 and K % 32 == 0 and K // 32 >= 64 and M * (K // 32) * 80 <= 48 * 1024


def assert_batch(items_np, M, seed, check_oracle=True):
    """items_np: list of (N, K, bits, x_key); items with the same x_key share x."""
    xs = {}
    items, meta = [], []
    for i, (N, K, bits, xk) in enumerate(items_np):
        if (xk, K) not in xs:
            xs[(xk, K)] = workload.activations(62, seed * 100 + xk + K, M, K)
        P, S, o_p, o_s = quantized(seed * 1000 + i, N, K, bits)
        items.append((bf16_gpu(xs[(xk, K)]), P, S, K, bits))
        meta.append((N, K, bits, xs[(xk, K)], o_p, o_s))
    report("gemv_batched M=%d items=%d seed=%d" % (M, len(items), seed))
    ys = dq.gemv_batched(items)
    again = dq.gemv_batched(items)
    singles = [dq.gemv(x, P, S, K, b) for (x, P, S, K, b) in items]
    torch().cuda.synchronize()
    for i, ((N, K, bits, x, o_p, o_s), y, y2, y1) in enumerate(zip(meta, ys, again, singles)):
        assert np.array_equal(f32_bits(y), f32_bits(y2)), "item %d not deterministic" % i
        if not streamed(M, K):
            assert np.array_equal(f32_bits(y), f32_bits(y1)), "item %d differs from dq_gemv" % i
        if check_oracle:
            y_ref, bound = oracle.matmul(x, o_p, o_s, N, K, bits)
            assert within_tolerance(y.cpu().numpy(), y_ref, bound).all(), "item %d" % i


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_batched_mixed_widths(M):
    items = [(N, K, b, i % 3) for i, (N, K, b) in enumerate(MIXED)]
    assert_batch(items, M, seed=M)


@pytest.mark.parametrize("M", [1, 2, 8, 16])
def test_batched_stream_row_boundaries(M):
    """M <= 2: streamed rows that end inside a slice (65, 160, 544 chunks),
    exactly a slice (64), whole slices (2048 and 4096 codes), many rows per
    wave next to few, ragged last workgroups.  M >= 3: the same items as
    16- and 32-row tiles (ragged last tiles), bit for bit as dq_gemv."""
    items = [(1000, 2048, 6, 0), (77, 2080, 5, 1), (3, 5120, 7, 2), (4097, 5120, 4, 2),
             (250, 17408, 8, 3), (513, 4096, 15, 4), (2, 2080, 2, 1), (1, 4096, 9, 4)]
    assert_batch(items, M, seed=50 + M)


@pytest.mark.parametrize("M", [1, 16])
def test_batched_largest_batch_and_one_item(M):
    items = [(N, K, b, 0) for (N, K, b) in MIXED] * 3
    assert_batch(items[:dq.GEMV_BATCH_MAX], M, seed=40)
    assert_batch(items[:1], M, seed=41)
    if M == 1:
        assert_batch([(3, 1 << 22, 5, 0), (70, 2048, 6, 0)], M, seed=42)  # x too large for LDS


def test_batched_decode_workload():
    """The decode workload's five 4096 x 4096 matrices (b = 4 .. 8, one
    activation) as one launch: the same bits on every call, sampled rows
    within the tolerance of the oracle."""
    N = K = 4096
    x = workload.activations(2, 0, 1, K)
    X = bf16_gpu(x)
    items, w_rows = [], []
    rows = np.random.default_rng(3).choice(N, 64, replace=False)
    for b in (4, 5, 6, 7, 8):
        w = workload.weights(2, b, N, K, outlier_frac=0.001)
        P, S = dq.quantize_pack(weights_gpu(w), b)
        items.append((X, P, S, K, b))
        w_rows.append(w[rows])
    report("gemv_batched decode workload")
    ys = dq.gemv_batched(items)
    again = dq.gemv_batched(items)
    torch().cuda.synchronize()
    for (X_, P, S, K_, b), y, y2, wr in zip(items, ys, again, w_rows):
        assert np.array_equal(f32_bits(y), f32_bits(y2))
        o_p, o_s = oracle_rows(wr, rows, P, S, b)
        y_ref, bound = oracle.matmul(x, o_p, o_s, len(rows), K, b)
        assert within_tolerance(y.cpu().numpy()[:, rows], y_ref, bound).all()


@pytest.mark.parametrize("M", [1, 8])
def test_batched_layer_shapes(M):
    """One layer of the 448-matrix stack (4 x 5120^2, 2 x 17408 x 5120,
    5120 x 17408) at widths 5 .. 8 in one call: the same bits on every call,
    sampled rows against the oracle; at M = 8 the same bits as dq_gemv."""
    t = torch()
    shapes = [(5120, 5120, 6), (5120, 5120, 5), (5120, 5120, 6), (5120, 5120, 7),
              (17408, 5120, 6), (17408, 5120, 8), (5120, 17408, 5)]
    g = t.Generator(device="cuda")
    g.manual_seed(7)
    items, W_rows = [], {}
    for i, (N, K, b) in enumerate(shapes):
        W = (t.randn((N, K), generator=g, device="cuda") * 0.02).to(t.bfloat16)
        P, S = dq.quantize_pack(W, b)
        rows = np.random.default_rng(K + b).choice(N, 32, replace=False)
        # the sampled rows' bf16 bits, for the oracle
        W_rows[(K, b, P.data_ptr())] = W.index_select(0, t.from_numpy(rows).cuda()).view(t.int16) \
            .cpu().numpy().view(np.uint16)
        x = workload.activations(63, i, M, K)
        items.append((bf16_gpu(x), P, S, K, b, x))
        del W
    report("gemv_batched layer shapes M=%d" % M)
    ys = dq.gemv_batched([it[:5] for it in items])
    again = dq.gemv_batched([it[:5] for it in items])
    singles = [dq.gemv(X, P, S, K, b) for (X, P, S, K, b, _) in items] if M > 2 else ys
    t.cuda.synchronize()
    for (X, P, S, K, b, x), y, y2, y1 in zip(items, ys, again, singles):
        assert np.array_equal(f32_bits(y), f32_bits(y2))
        assert np.array_equal(f32_bits(y), f32_bits(y1))
        rows = np.random.default_rng(K + b).choice(P.shape[0], 32, replace=False)
        o_p, o_s = oracle_rows(W_rows[(K, b, P.data_ptr())], rows, P, S, b)
        y_ref, bound = oracle.matmul(x, o_p, o_s, len(rows), K, b)
        assert within_tolerance(y.cpu().numpy()[:, rows], y_ref, bound).all()


# (N, K, bits, scheme, group): scheme "a" zero points, "g" group scales, "s"
# symmetric; the row-sliced bodies (one and two rows per slice), the
# resident-x body, wide codes and items that take a launch of their own
VARIANTS = [(200, 4096, 5, "a", 0), (130, 5120, 7, "a", 0), (64, 1024, 4, "a", 0),
            (50, 2080, 6, "a", 0), (20, 4096, 12, "a", 0), (91, 3072, 8, "a", 0),
            (200, 4096, 6, "g", 128), (130, 5120, 5, "g", 64), (64, 1024, 8, "g", 256),
            (50, 2080, 6, "g", 32), (40, 6144, 9, "g", 2048), (33, 4096, 15, "g", 32),
            (9, 4133, 6, "a", 0), (9, 4133, 7, "g", 64),  # K not a multiple of 32
            (300, 4096, 6, "s", 0), (77, 2080, 5, "s", 0)]


def variant_weights(seed, N, K, scheme):
    """bf16 weights: for zero points, rows moved off zero (every fifth
    non-negative) with every third row sparse -- one positive element, the rest
    zero (z = 0), where a fold through sum_k x would cancel; returns the
    weights and the sparse rows' non-zero positions."""
    rng = np.random.default_rng(seed)
    wf = workload.bf16_to_f32(workload.weights(65, seed, N, K, dtype="bf16"))
    pos = {}
    if scheme == "a":
        wf = wf + rng.uniform(-0.04, 0.04, N).astype(np.float32)[:, None]
        wf[::5] = np.abs(wf[::5])
        for n in range(1, N, 3):
            p = int(rng.integers(0, K))
            v = abs(float(wf[n, p])) + 0.01
            wf[n] = 0.0
            wf[n, p] = v
            pos[n] = p
    return workload.bf16_from_f32(wf.astype(np.float32)), pos


@pytest.mark.parametrize("M", [1, 2, 8])
def test_batched_zero_points_and_group_scales(M):
    """Items with zero points and with group scales beside symmetric ones in
    one call (one launch per scheme at M <= 2; at M = 8 the variant items run
    one launch each beside the symmetric items' one): each output within the bar of the
    oracle's own product (sparse asymmetric rows with small activations at
    their one non-zero included), the same bits on every call, and the same
    bits as the scheme's one-matrix entry point for the items that do not
    stream."""
    t = torch()
    items, meta = [], []
    for i, (N, K, bits, scheme, g) in enumerate(VARIANTS):
        seed = 7000 + 100 * M + i
        w, pos = variant_weights(seed, N, K, scheme)
        x = workload.activations(66, seed, M, K)
        if pos:  # small activations at the sparse rows' non-zeros
            cols = np.array(sorted(set(pos.values())))
            xf = workload.bf16_to_f32(x)
            rng = np.random.default_rng(seed)
            xf[:, cols] = (rng.uniform(0.005, 0.05, (M, len(cols))) *
                           rng.choice([-1.0, 1.0], (M, len(cols)))).astype(np.float32)
            x = workload.bf16_from_f32(xf)
        X = bf16_gpu(x)
        if scheme == "a":
            o_p, o_s, o_z, _ = oracle.quantize_pack_asym(w, bits)
            Z = t.from_numpy(o_z).cuda()
            item = (X, t.from_numpy(o_p.view(np.int32)).cuda(), t.from_numpy(o_s).cuda(), K, bits, Z)
            ref = oracle.matmul_asym(x, o_p, o_s, o_z, N, K, bits)
        elif scheme == "g":
            o_p, o_s, _ = oracle.quantize_pack_group(w, bits, g)
            item = (X, t.from_numpy(o_p.view(np.int32)).cuda(), t.from_numpy(o_s).cuda(), K, bits, None, g)
            ref = oracle.matmul_group(x, o_p, o_s, N, K, bits, g)
        else:
            o_p, o_s, _ = oracle.quantize_pack(w, bits)
            item = (X, t.from_numpy(o_p.view(np.int32)).cuda(), t.from_numpy(o_s).cuda(), K, bits)
            ref = oracle.matmul(x, o_p, o_s, N, K, bits)
        items.append(item)
        meta.append((N, K, bits, scheme, g, ref))
    report("gemv_batched schemes M=%d items=%d" % (M, len(items)))
    ys = dq.gemv_batched(items)
    again = dq.gemv_batched(items)
    singles = []
    for (X, P, S, K, bits, *rest), (_, _, _, scheme, g, _) in zip(items, meta):
        if scheme == "a":
            singles.append(dq.gemv_asym(X, P, S, rest[0], K, bits))
        elif scheme == "g":
            singles.append(dq.gemv_group(X, P, S, K, bits, g))
        else:
            singles.append(dq.gemv(X, P, S, K, bits))
    t.cuda.synchronize()
    for i, ((N, K, bits, scheme, g, (y_ref, bound)), y, y2, y1) in enumerate(zip(meta, ys, again, singles)):
        assert np.array_equal(f32_bits(y), f32_bits(y2)), "item %d not deterministic" % i
        nch = K // 32
        fits = K % 32 == 0 and M * nch * 80 <= 48 * 1024
        streams = M <= 2 and fits and nch >= 64 and (nch % 32 == 0 if scheme != "s" else True)
        if not streams:
            assert np.array_equal(f32_bits(y), f32_bits(y1)), "item %d differs from its entry point" % i
        ok = within_tolerance(y.cpu().numpy(), y_ref, bound)
        assert ok.all(), "item %d (%s b=%d N=%d K=%d g=%d): %d outputs out of tolerance" % (
            i, scheme, bits, N, K, g, int((~ok).sum()))
