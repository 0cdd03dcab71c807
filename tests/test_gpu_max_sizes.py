"""Products at the largest shapes the kernels treat differently: a weight
matrix of 2^22 + 96 rows, so that one 256-row tile of the GEMM's output spans
more than 4 GiB (the wide kernel's unchecked buffer stores stop at 4 GiB and
the checked per-element stores take over), through dq_gemm (M = 300: a ragged
last row tile), dq_gemv (M = 1 and 8) and the batched launch.  The codes are
seeded random words (every code value 0 .. 2^b - 1 occurs, the extremes
included) and the outputs are checked against the oracle on sampled entries
(the first, the last and random rows and columns), to the usual bar."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, report, torch
from pins import within_tolerance

pytestmark = pytest.mark.gpu

N = (1 << 22) + 96
K = 64


def sampled_check(y_dev, x, packed_np, scales_np, bits, seed, tag):
    t = torch()
    M = x.shape[0]
    rng = np.random.default_rng([41, seed])
    ns = np.unique(np.concatenate([[0, 1, N - 97, N - 96, N - 1], rng.integers(0, N, 200)]))
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    got = y_dev[t.from_numpy(mm.ravel()).cuda(), t.from_numpy(nn.ravel()).cuda()].cpu().numpy()
    y_ref, bound = oracle.matmul_pairs(x, packed_np, scales_np, N, K, bits, mm.ravel(), nn.ravel())
    ok = within_tolerance(got, y_ref, bound)
    if not ok.all():
        i = int(np.argmin(ok))
        pytest.fail("%s: y[%d,%d]=%r ref %r bound %r (%d bad)" % (
            tag, mm.ravel()[i], nn.ravel()[i], got[i], y_ref[i], bound[i], int((~ok).sum())))


@pytest.mark.parametrize("bits", [3, 12])
def test_products_with_four_gib_output_tiles(bits):
    t = torch()
    g = t.Generator(device="cuda")
    g.manual_seed(4200 + bits)
    rw = dq.packed_row_bytes(K, bits) // 4
    report("max-size products: N=%d K=%d bits=%d (%.2f GB of codes)" % (N, K, bits, N * rw * 4 / 1e9))
    P = t.randint(-(1 << 31), (1 << 31) - 1, (N, rw), dtype=t.int32, device="cuda", generator=g)
    used = (K * bits + 31) // 32  # padding words past the codes stay zero
    P[:, used:] = 0
    S = (t.rand(N, device="cuda", generator=g) * 1e-3 + 1e-5).float()
    packed_np = P.cpu().numpy().view(np.uint32)
    scales_np = S.cpu().numpy()
    for M, fn in ((300, dq.gemm), (1, dq.gemv), (8, dq.gemv)):
        x = workload.activations(42, bits * 10 + M, M, K)
        tag = "%s M=%d N=%d K=%d bits=%d" % (fn.__name__, M, N, K, bits)
        report(tag)
        y = fn(bf16_gpu(x), P, S, K, bits)
        t.cuda.synchronize()
        sampled_check(y, x, packed_np, scales_np, bits, bits * 10 + M, tag)
        del y
    x = workload.activations(42, bits * 10 + 2, 1, K)
    report("gemv_batched M=1 N=%d bits=%d" % (N, bits))
    (y,) = dq.gemv_batched([(bf16_gpu(x), P, S, K, bits)])
    t.cuda.synchronize()
    sampled_check(y, x, packed_np, scales_np, bits, bits * 10 + 2, "batched")
