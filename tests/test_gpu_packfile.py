"""The on-disk packed-weight format on the GPU: matrices quantized on the
GPU, written to a file, mapped and copied back into device memory come back
bit for bit, and the GEMV on the loaded buffers gives the same bits as on the
originals (and agrees with the oracle).  The BF16 level (16: weights kept)
round-trips as bf16.

Source: DynaQuant page (zingnex.cn), "项目现状与路线图" (packed-weight format
on disk); "第三步：应用配方" (a recipe applied per matrix)."""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
import oracle
import workload
from gpu_util import bf16_gpu, f32_bits, report, torch, u32, weights_gpu
from pins import within_tolerance

pytestmark = pytest.mark.gpu


def test_recipe_round_trip(tmp_path):
    recipe = [(300, 640, 5), (257, 1000, 6), (64, 4096, 8), (33, 96, 12), (40, 72, 16), (129, 2048, 3)]
    ws = [workload.weights(3, 200 + i, n, k) for i, (n, k, _) in enumerate(recipe)]
    mats, dev = [], []
    for i, ((n, k, b), w_np) in enumerate(zip(recipe, ws)):
        report("packed file: quantize matrix %d %dx%d b=%d" % (i, n, k, b))
        if b == 16:
            mats.append(("m%d" % i, n, k, 16, w_np, None))
            dev.append(None)
            continue
        packed, scales = dq.quantize_pack(weights_gpu(w_np), b)
        torch().cuda.synchronize()
        mats.append(("m%d" % i, n, k, b, u32(packed), scales.cpu().numpy()))
        dev.append((packed, scales))
    path = str(tmp_path / "recipe.dqw")
    dq.write_packed_file(path, mats)
    with dq.PackedFile(path) as pf:
        assert len(pf) == len(recipe)
        for i, ((n, k, b), w_np) in enumerate(zip(recipe, ws)):
            assert pf.verify(i)
            report("packed file: load matrix %d" % i)
            data, scales = pf.load(i)
            if b == 16:
                assert data.dtype == torch().bfloat16
                assert np.array_equal(data.cpu().view(torch().int16).numpy().view(np.uint16), w_np)
                continue
            packed, s0 = dev[i]
            assert np.array_equal(u32(data), u32(packed))
            assert np.array_equal(f32_bits(scales), f32_bits(s0))
            o_packed, o_scales, _ = oracle.quantize_pack(w_np, b)
            assert np.array_equal(u32(data), o_packed)
            x_np = workload.activations(3, 200 + i, 4, k)
            x = bf16_gpu(x_np)
            y_loaded = dq.gemv(x, data, scales, k, b)
            y_orig = dq.gemv(x, packed, s0, k, b)
            torch().cuda.synchronize()
            assert y_loaded.cpu().numpy().tobytes() == y_orig.cpu().numpy().tobytes()
            y_ref, bound = oracle.matmul(x_np, o_packed, o_scales, n, k, b)
            assert within_tolerance(y_loaded.cpu().numpy(), y_ref, bound).all()
