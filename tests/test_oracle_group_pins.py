"""Pins of the oracle's group-wise quantizer, and a mutation check on a copy of
its C source.  The group-wise scheme applies the pinned per-row quantizer to
every group of g consecutive weights of a row, so the strongest pin is that
reduction itself: quantizing W[N, K] with groups of g must give exactly the
per-row quantizer's codes and scales on the [N*K/g, g] matrix of groups.

Source: "量化" tutorial (aiknowledge.cn), exercise 1 of its exercises
section (one scale per group of weights, group sizes 32 to 256, as GPTQ/AWQ
use, instead of one per channel)."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload

SRC = os.path.join(os.path.dirname(oracle.__file__), "dq_oracle.c")


def check_reduces_to_rows(orc) -> list[str]:
    bad = []
    for bits in (2, 4, 6, 9, 15):
        for g in (32, 64, 128, 256):
            N, K = 5, 4 * g
            w = workload.weights(41, bits * 10 + g, N, K, outlier_frac=0.01)
            if g == 64:
                w[1, g:2 * g] = 0  # an all-zero group
            packed, scales, q = orc.quantize_pack_group(w, bits, g)
            p_rows, s_rows, q_rows = orc.quantize_pack(w.reshape(N * K // g, g), bits)
            if not np.array_equal(q.reshape(-1, g), q_rows):
                bad.append("b=%d g=%d codes differ from the per-row quantizer" % (bits, g))
            if not np.array_equal(scales.reshape(-1).view(np.uint32), s_rows.view(np.uint32)):
                bad.append("b=%d g=%d scales differ from the per-row quantizer" % (bits, g))
            if not np.array_equal(packed, orc.pack(q, bits)):
                bad.append("b=%d g=%d packing" % (bits, g))
    return bad


def check_ragged_and_single_group(orc) -> list[str]:
    """K not a multiple of g: the last, shorter group is quantized as a row of
    its own length; g >= K is the per-row quantizer."""
    bad = []
    for bits in (3, 8, 12):
        N, K, g = 4, 300, 128
        w = workload.weights(42, bits, N, K, dtype="f32")
        w[2, 260] = np.nan  # a non-finite element poisons only its own group
        packed, scales, q = orc.quantize_pack_group(w, bits, g)
        if scales.shape != (N, 3):
            bad.append("b=%d group count" % bits)
        for j, (k0, k1) in enumerate(((0, 128), (128, 256), (256, 300))):
            _, s_ref, q_ref = orc.quantize_pack(np.ascontiguousarray(w[:, k0:k1]), bits)
            if not (np.array_equal(q[:, k0:k1], q_ref)
                    and np.array_equal(scales[:, j].view(np.uint32), s_ref.view(np.uint32))):
                bad.append("b=%d group %d" % (bits, j))
        if not (np.isnan(scales[2, 2]) and np.isfinite(scales[2, :2]).all()):
            bad.append("b=%d non-finite group" % bits)
        p1, s1, q1 = orc.quantize_pack_group(w[:, :100].copy(), bits, 128)
        p2, s2, q2 = orc.quantize_pack(w[:, :100].copy(), bits)
        if not (np.array_equal(p1, p2) and np.array_equal(s1[:, 0], s2) and np.array_equal(q1, q2)):
            bad.append("b=%d single group" % bits)
    return bad


def check_unpack_and_matmul(orc) -> list[str]:
    bad = []
    for bits in (2, 5, 10):
        N, K, g = 3, 70, 32
        w = workload.weights(43, bits, N, K, dtype="f32")
        w[:, 32:64] *= 50  # groups of very different magnitude
        packed, scales, q = orc.quantize_pack_group(w, bits, g)
        q2, w_hat = orc.unpack_group(packed, scales, N, K, bits, g)
        if not np.array_equal(q2, q):
            bad.append("b=%d unpack codes" % bits)
        for n in range(N):
            for k in range(K):
                if w_hat[n, k] != np.float32(np.float32(q[n, k]) * scales[n, k // g]):
                    bad.append("b=%d dequant (%d,%d)" % (bits, n, k))
                    break
        x = workload.activations(43, bits, 2, K)
        xf = workload.bf16_to_f32(x)
        y, bound = orc.matmul_group(x, packed, scales, N, K, bits, g)
        for m in range(2):
            for n in range(N):
                terms = [Fraction(float(xf[m, k])) * int(q[n, k]) * Fraction(float(scales[n, k // g]))
                         for k in range(K)]
                if y[m, n] != float(sum(terms)) or bound[m, n] != float(sum(abs(t) for t in terms)):
                    bad.append("b=%d matmul (%d,%d)" % (bits, m, n))
        onehot = np.zeros((1, K), np.uint16)
        onehot[0, 40] = 0x3F80
        y, _ = orc.matmul_group(onehot, packed, scales, N, K, bits, g)
        if not np.array_equal(y[0].astype(np.float32), w_hat[:, 40]):
            bad.append("b=%d one-hot" % bits)
    return bad


CHECKS = [check_reduces_to_rows, check_ragged_and_single_group, check_unpack_and_matmul]


def run_all(orc) -> list[str]:
    bad = []
    for c in CHECKS:
        bad += c(orc)
    return bad


@pytest.mark.parametrize("check", CHECKS)
def test_group_oracle_pinned(check):
    assert check(oracle.default()) == []


MUTANTS = [
    ("group_count_floor", "const int64_t G = (K + g - 1) / g;\n#pragma omp parallel for schedule(dynamic, 16)\n"
     "    for (int64_t n = 0; n < N; n++) {\n        int32_t *q = (int32_t *)malloc((size_t)K * sizeof *q);\n"
     "        float *piece",
     "const int64_t G = K / g;\n#pragma omp parallel for schedule(dynamic, 16)\n"
     "    for (int64_t n = 0; n < N; n++) {\n        int32_t *q = (int32_t *)malloc((size_t)K * sizeof *q);\n"
     "        float *piece"),
    ("last_group_short", "int64_t k0 = j * g, len = (K - k0 < g) ? K - k0 : g;",
     "int64_t k0 = j * g, len = (K - k0 < g) ? K - k0 - 1 : g;"),
    ("unpack_scale_of_row", "w_out[n * K + k] = (float)q[k] * scales[n * G + k / g];",
     "w_out[n * K + k] = (float)q[k] * scales[n * G];"),
    ("matmul_scale_index_mod", "(double)scales[n * G + k / g];", "(double)scales[n * G + k % G];"),
    ("matmul_bound_signed", "total_abs += fabs(term);", "total_abs += term;"),
    ("groups_share_first_scale", "quantize_row(piece, 0, 0, len, bits, q + k0, &scales[n * G + j]);",
     "quantize_row(piece, 0, 0, len, bits, q + k0, &scales[n * G + j]);\n"
     "            if (j > 0) scales[n * G + j] = scales[n * G];"),
]


def test_group_pins_accept_the_oracle():
    assert run_all(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_group_pins_reject_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique/found: %s" % name
    mut = tmp_path / ("oracle_%s.c" % name)
    mut.write_text(src.replace(old, new))
    path = oracle.build(force=True, src=str(mut), out=str(tmp_path / ("lib_%s.so" % name)))
    try:
        bad = run_all(oracle.Oracle(path))
    except Exception as e:  # a mutant may also crash a check outright
        bad = ["raised %r" % e]
    assert bad, "mutant %s passed every pin" % name
