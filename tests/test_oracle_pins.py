"""Pins of the CPU oracle against what the pages and the mathematics fix.

Runs without a GPU.  Sources: "量化" (Quantization) tutorial, aiknowledge.cn
("how quantization works", "Step 1" per-channel quantizer, "Step 7" memory
calculator); DynaQuant page, zingnex.cn (results table, custom kernel
architecture, pack/unpack utilities); BPDQ article, section 3.2 (fused
dequantize + matmul).
"""
from __future__ import annotations

import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload
from pins import (F32_QNAN_BITS, check_matmul_exact, check_pack, check_quantize_invariants,
                  check_quantize_row, f32_bits, row_bytes_formula, stream_words)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- fixtures

def parse_examples(path):
    blocks, cur = [], None
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        m = re.match(r"\[(\w+)\]$", line)
        if m:
            cur = {"name": m.group(1)}
            blocks.append(cur)
            continue
        k, v = (p.strip() for p in line.split("=", 1))
        cur[k] = v
    return blocks


EXAMPLES = parse_examples(os.path.join(GOLDEN, "quantize_examples.txt"))


def as_input(values, dtype):
    f = np.array(values, dtype=np.float32)[None, :]
    if dtype == "f32":
        return f, f
    bits = workload.bf16_from_f32(f)
    assert np.array_equal(workload.bf16_to_f32(bits), f), "example value not exact in bf16"
    return bits, f


@pytest.mark.parametrize("ex", EXAMPLES, ids=[e["name"] for e in EXAMPLES])
def test_golden_example(ex):
    bits = int(ex["bits"])
    w_in, w_f32 = as_input([float(v) for v in ex["w"].split()], ex["dtype"])
    packed, scales, q = oracle.quantize_pack(w_in, bits)
    assert "%08x" % f32_bits(scales[0]) == ex["scale_hex"]
    assert q[0].tolist() == [int(v) for v in ex["q"].split()]
    want = [int(v) for v in ex["words"].split()]
    assert packed.shape[1] == 32  # every example fits one 128-byte row
    assert packed[0, :len(want)].tolist() == want
    assert not packed[0, len(want):].any()
    assert check_quantize_row(w_f32[0], bits, q[0], scales[0]) == []


def test_byte_model_against_pages():
    rows = []
    for line in open(os.path.join(GOLDEN, "byte_model.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            src, p, b, gb, dec = line.split()
            rows.append((src, float(p), float(b), float(gb), int(dec)))
    for src, p, b, gb, dec in rows:
        if src == "calc":
            model = p * 1e9 * b / 8 / 1e9  # params * bits / 8, decimal GB
            assert np.floor(model * 10 ** dec + 1e-9) / 10 ** dec == gb, (p, b, gb)
        else:
            # same parameters at b bits instead of 16; the page's inputs are
            # printed to one decimal, so the model is an interval
            lo = (p - 0.05) * (b - 0.05) / 16.0
            hi = (p + 0.05) * (b + 0.05) / 16.0
            assert lo <= gb + 0.05 and gb - 0.05 <= hi, (p, b, gb)
            assert lo <= p * b / 16.0 <= hi


@pytest.mark.parametrize("bits", range(2, 16))
def test_packed_bytes_equal_bits_times_params(bits):
    # rows of 5120 and 17408 codes are whole multiples of 128 bytes at every b,
    # so the packed size of a matrix is exactly params * bits / 8
    for N, K in workload.stack_shapes()[:7]:
        assert N * oracle.row_bytes(K, bits) * 8 == N * K * bits
    # the 448-matrix stack at its per-matrix recipe
    shapes, recipe = workload.stack_shapes(), workload.stack_bits()
    total = sum(N * oracle.row_bytes(K, b) for (N, K), b in zip(shapes, recipe))
    assert total * 8 == sum(N * K * b for (N, K), b in zip(shapes, recipe))


def test_row_bytes_formula():
    for bits in range(2, 16):
        for K in list(range(1, 300)) + [614, 1000, 4095, 4096, 4097, 8192, 17408]:
            rb = oracle.row_bytes(K, bits)
            assert rb == row_bytes_formula(K, bits)
            assert rb % 128 == 0 and rb * 8 >= K * bits and (rb - 128) * 8 < K * bits


# ------------------------------------------------------------ quantizer

def brute_rows(bits, rng):
    """Random and constructed rows (fp32) that exercise every branch."""
    qmax = (1 << (bits - 1)) - 1
    rows = []
    for K in (1, 2, 3, 7, 16, 24):
        rows.append(rng.standard_normal(K).astype(np.float32) * np.float32(0.02))
    # a row hitting every level exactly: w = j * s0 with s0 a power of two
    s0 = np.float32(2.0 ** -6)
    levels = np.arange(-qmax, qmax + 1, max(1, (2 * qmax) // 24), dtype=np.int64)
    levels = np.unique(np.concatenate([levels, [qmax, -qmax, 0, 1, -1]]))
    rows.append((levels * s0).astype(np.float32))
    # exact ties (j + 1/2) * s0 with absmax = qmax * s0
    j = np.arange(-min(qmax, 6), min(qmax, 6)).astype(np.float64)
    tie = np.concatenate([[qmax], j + 0.5]) * float(s0)
    rows.append(tie.astype(np.float32))
    rows.append(np.array([-0.0, 0.0, -0.0], np.float32))  # zero row, signed zeros
    rows.append(np.array([0.7, 0.7, -0.7], np.float32))  # constant magnitude
    rows.append(np.array([3e-39, -1e-39, 5e-45], np.float32))  # subnormal absmax
    rows.append(np.array([1.4e-45, -1.4e-45, 0.0], np.float32))  # smallest subnormal
    rows.append(np.array([3.0e38, -1.0e38, 1.0], np.float32))  # near the top of the range
    rows.append(np.array([0.5, -2.0 ** -30, 2.0 ** -20], np.float32))  # wide dynamic range
    return rows


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_brute_force(bits):
    rng = np.random.default_rng(1000 + bits)
    for w in brute_rows(bits, rng):
        packed, scales, q = oracle.quantize_pack(w[None, :], bits)
        assert check_quantize_row(w, bits, q[0], scales[0]) == [], (bits, w)


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_brute_force_bf16(bits):
    rng = np.random.default_rng(2000 + bits)
    w = workload.bf16_from_f32(rng.standard_normal((6, 20)).astype(np.float32) * np.float32(0.02))
    packed, scales, q = oracle.quantize_pack(w, bits)
    wf = workload.bf16_to_f32(w)
    for n in range(w.shape[0]):
        assert check_quantize_row(wf[n], bits, q[n], scales[n]) == []


def test_nonfinite_rows():
    w = np.array([[1.0, np.nan, 0.5], [np.inf, 0.1, 0.2], [0.1, -np.inf, 0.0], [0.3, 0.2, 0.1]],
                 np.float32)
    for bits in (2, 6, 15):
        packed, scales, q = oracle.quantize_pack(w, bits)
        for n in range(3):
            assert f32_bits(scales[n]) == F32_QNAN_BITS
            assert not q[n].any()
        assert check_quantize_row(w[3], bits, q[3], scales[3]) == []
        for n in range(4):
            assert check_quantize_row(w[n], bits, q[n], scales[n]) == []


@pytest.mark.parametrize("bits", range(2, 16))
def test_quantize_invariants(bits):
    w = workload.weights(99, bits, 64, 1000, outlier_frac=0.001, dtype="f32")
    w[5] = 0
    packed, scales, q = oracle.quantize_pack(w, bits)
    assert check_quantize_invariants(w, bits, q, scales) == []
    wt = workload.weights(98, bits, 32, 777, dist="t5")
    packed, scales, q = oracle.quantize_pack(wt, bits)
    assert check_quantize_invariants(workload.bf16_to_f32(wt), bits, q, scales) == []


def test_page_per_channel_formula_b8():
    """Cross-check (not a pin): at the tutorial's default width of 8 bits the
    per-channel routine of its Step 1, reducing over each row in fp32, gives
    the same scales and codes."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((50, 300)) * 0.02).astype(np.float32)
    w[3] = 0
    qmax = 2 ** 7 - 1
    abs_max = np.max(np.abs(w), axis=1, keepdims=True)
    scales = np.where(abs_max == 0, np.float32(1.0), abs_max) / np.float32(qmax)
    want_q = np.clip(np.round(w / scales), -qmax - 1, qmax).astype(np.int32)
    packed, s, q = oracle.quantize_pack(w, 8)
    assert np.array_equal(q, want_q)
    assert np.array_equal(s, scales.squeeze().astype(np.float32))


# --------------------------------------------------------------- packing

@pytest.mark.parametrize("bits", range(2, 16))
def test_pack_matches_big_integer_stream(bits):
    rng = np.random.default_rng(3000 + bits)
    lim = 1 << (bits - 1)
    for K in (1, 5, 31, 32, 33, 100, 614):
        q = rng.integers(-lim, lim, size=(3, K), dtype=np.int32)
        q[0, 0], q[0, -1] = -lim, lim - 1  # codes 0 and 2^b - 1
        packed = oracle.pack(q, bits)
        assert check_pack(q, bits, packed) == []
        q2, _ = oracle.unpack(packed, None, 3, K, bits)
        assert np.array_equal(q2, q)


@pytest.mark.parametrize("bits", [2, 5, 8, 11, 15])
def test_quantize_pack_unpack_roundtrip(bits):
    w = workload.weights(97, bits, 40, 333)
    packed, scales, q = oracle.quantize_pack(w, bits)
    assert check_pack(q, bits, packed) == []
    q2, w_hat = oracle.unpack(packed, scales, 40, 333, bits)
    assert np.array_equal(q2, q)
    # dequantized weight = fl32(q * s): numpy's fp32 multiply, bit for bit
    want = q.astype(np.float32) * scales[:, None]
    assert np.array_equal(w_hat.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- matmul

@pytest.mark.parametrize("bits", [2, 4, 7, 10, 15])
def test_matmul_exact_rational(bits):
    rng = np.random.default_rng(4000 + bits)
    M, N, K = 3, 4, 9
    w = workload.bf16_from_f32(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    x = workload.bf16_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    packed, scales, q = oracle.quantize_pack(w, bits)
    y, bound = oracle.matmul(x, packed, scales, N, K, bits)
    assert check_matmul_exact(workload.bf16_to_f32(x), q, scales, y, bound) == []


def test_matmul_closed_forms():
    bits, N, K = 6, 5, 11
    rng = np.random.default_rng(5)
    w = workload.bf16_from_f32(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    w[2] = 0
    w[4] = workload.bf16_from_f32(np.full(K, 0.25, np.float32))  # constant row
    packed, scales, q = oracle.quantize_pack(w, bits)
    onehot = np.zeros((K, K), np.float32)
    onehot[np.arange(K), np.arange(K)] = 1
    y, bound = oracle.matmul(workload.bf16_from_f32(onehot), packed, scales, N, K, bits)
    # one-hot row k picks column k: y = s[n] * q[n, k] exactly
    assert np.array_equal(y, (scales[None, :].astype(np.float64) * q.T))
    assert not y[:, 2].any() and not bound[:, 2].any()
    ones = workload.bf16_from_f32(np.ones((1, K), np.float32))
    y1, _ = oracle.matmul(ones, packed, scales, N, K, bits)
    qmax = 31
    assert y1[0, 4] == float(scales[4]) * qmax * K  # s * qmax * K


def test_matmul_pairs_match_full():
    bits, M, N, K = 9, 4, 6, 70
    w = workload.weights(96, 0, N, K)
    x = workload.activations(96, 0, M, K)
    packed, scales, q = oracle.quantize_pack(w, bits)
    y, bound = oracle.matmul(x, packed, scales, N, K, bits)
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    yp, bp = oracle.matmul_pairs(x, packed, scales, N, K, bits, ms.ravel(), ns.ravel())
    assert np.array_equal(yp, y.ravel()) and np.array_equal(bp, bound.ravel())


def test_stream_words_helper_known_value():
    # the helper itself, on the hand-derived b=5 example
    assert stream_words([15, -15, 0, 2, -2, 8, 0, 7], 5, 2) == [820592703, 188]
    assert Fraction(1, 2) == Fraction(float(np.float32(0.15)) / float(np.float32(0.3)))
