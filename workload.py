"""Seeded synthetic inputs for the quantize / pack / dequant-matmul workloads.

Shared by the tests and the benchmark; used to feed both the GPU library and
the CPU oracle.  Holds no quantization, packing or matmul arithmetic: only
random draws, the fp32 -> bf16 input rounding and the workload shapes.

Recipe (every draw is reproducible from its integers):
* generator: numpy PCG64 seeded with SeedSequence([workload, matrix, role,
  block]); role 0 = weights, 1 = activations, 2 = outlier positions,
  3 = bit-width shuffle, 4 = Hessian traces; weights are drawn in blocks of
  1024 rows;
* weights: fp32 draws times the stated std (0.02), rounded to bf16 with
  round-half-to-even on the bit pattern (or kept fp32 where the workload says
  fp32); Student-t(5) draws are divided by sqrt(5/3) so the std is 0.02;
* outliers: a fraction of positions drawn without replacement over the whole
  matrix, multiplied by 20 in fp32 before the bf16 rounding;
* activations: bf16 N(0, 1) rounded the same way;
* Hessian traces (the model-dependent half of a sensitivity, which needs a
  trained model and calibration data): one log-normal draw per matrix,
  exp(N(0, 1)), so sensitivities spread over about two decades.

The shapes follow the pages' model sizes: the 27B-class layer (5120 hidden,
17408 MLP, 64 layers, 448 matrices) of the DynaQuant page's results table and
its knee allocation (283 matrices at 6 bits, 98 at 5, the rest at 7-8).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROLE_W, ROLE_X, ROLE_OUTLIER, ROLE_SHUFFLE, ROLE_HTRACE = 0, 1, 2, 3, 4
ROW_BLOCK = 1024


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (half-to-even on the bit pattern); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _draw_block(workload: int, matrix: int, block: int, rows: int, K: int, dist: str,
                std: float) -> np.ndarray:
    g = _rng(workload, matrix, ROLE_W, block)
    if dist == "normal":
        v = g.standard_normal((rows, K), dtype=np.float32)
        v *= np.float32(std)
    elif dist == "t5":
        v = g.standard_t(5, size=(rows, K)).astype(np.float32)
        v *= np.float32(std / np.sqrt(5.0 / 3.0))
    else:
        raise ValueError(dist)
    return v


def weights(workload: int, matrix: int, N: int, K: int, *, dist: str = "normal",
            std: float = 0.02, outlier_frac: float = 0.0, outlier_mul: float = 20.0,
            dtype: str = "bf16", threads: int = 8) -> np.ndarray:
    """W[N, K]: uint16 bf16 bits (dtype='bf16') or float32 (dtype='f32')."""
    nblocks = (N + ROW_BLOCK - 1) // ROW_BLOCK
    out = np.empty((N, K), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(b: int):
        r0 = b * ROW_BLOCK
        rows = min(ROW_BLOCK, N - r0)
        v = _draw_block(workload, matrix, b, rows, K, dist, std)
        if outlier_frac > 0:
            # positions are global; pick the ones that fall in this block
            lo, hi = r0 * K, (r0 + rows) * K
            sel = outlier_positions[(outlier_positions >= lo) & (outlier_positions < hi)] - lo
            v.reshape(-1)[sel] *= np.float32(outlier_mul)
        out[r0:r0 + rows] = bf16_from_f32(v) if dtype == "bf16" else v

    outlier_positions = None
    if outlier_frac > 0:
        count = int(round(outlier_frac * N * K))
        outlier_positions = np.sort(_rng(workload, matrix, ROLE_OUTLIER, 0).choice(
            N * K, size=count, replace=False))
    if nblocks == 1 or threads <= 1:
        for b in range(nblocks):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def activations(workload: int, matrix: int, M: int, K: int) -> np.ndarray:
    """x[M, K] as bf16 bits, N(0, 1)."""
    g = _rng(workload, matrix, ROLE_X, 0)
    return bf16_from_f32(g.standard_normal((M, K), dtype=np.float32))


def stack_bits(workload: int = 3) -> list[int]:
    """Per-matrix bit widths of the 448-matrix stack: 283 at 6, 98 at 5, 40 at 7 and
    27 at 8 (the DynaQuant knee allocation), shuffled with a seeded permutation."""
    bits = [6] * 283 + [5] * 98 + [7] * 40 + [8] * 27
    perm = _rng(workload, 0, ROLE_SHUFFLE, 0).permutation(len(bits))
    return [bits[i] for i in perm]


def hessian_traces(workload: int, count: int) -> np.ndarray:
    """Synthetic per-matrix Hessian traces: fp64 exp(N(0, 1)), one per matrix."""
    g = _rng(workload, 0, ROLE_HTRACE, 0)
    return np.exp(g.standard_normal(count))


def stack_shapes() -> list[tuple[int, int]]:
    """(N, K) of the 448 matrices in layer order: 4 attention projections
    5120x5120, gate and up 17408x5120, down 5120x17408, for 64 layers."""
    layer = [(5120, 5120)] * 4 + [(17408, 5120), (17408, 5120), (5120, 17408)]
    return layer * 64


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: weight shape and distribution, bit widths, M values."""
    index: int
    name: str
    N: int
    K: int
    bits: tuple
    gemv_m: tuple = ()
    gemm_m: tuple = ()
    dist: str = "normal"
    dtype: str = "bf16"
    outlier_frac: float = 0.0
    notes: str = field(default="", compare=False)


WORKLOADS = {
    1: Workload(1, "single-matrix-256", 256, 256, (6,), gemv_m=(1,), dtype="f32",
                notes="fp32 W ~ N(0, 0.02^2), b=6, x 1x256"),
    2: Workload(2, "decode-gemv-4096", 4096, 4096, (4, 5, 6, 7, 8), gemv_m=(1,),
                outlier_frac=0.001, notes="bf16 W with 0.1% outliers x20, x 1x4096"),
    3: Workload(3, "stack-448", 0, 0, (5, 6, 7, 8), gemv_m=(1, 8),
                notes="64 layers x 7 matrices, knee allocation, GEMV over every matrix"),
    4: Workload(4, "prefill-gemm-8192", 8192, 8192, (5, 6, 8, 12), gemm_m=(2048,),
                notes="bf16 W, x 2048x8192, fp32 y"),
    5: Workload(5, "sweep-28672x8192", 28672, 8192, tuple(range(2, 16)), gemv_m=(1, 16),
                gemm_m=(256,), dist="t5", notes="Student-t(5) W scaled to std 0.02"),
}


def workload_weights(w: Workload, matrix: int, **kw) -> np.ndarray:
    return weights(w.index, matrix, w.N, w.K, dist=w.dist, outlier_frac=w.outlier_frac,
                   dtype=w.dtype, **kw)
