"""Pins of the oracle's asymmetric (zero-point) quantizer, and a mutation check
that plants mistakes in a copy of its C source.  None of the pins re-runs the
oracle's arithmetic: they use closed forms, exact rational arithmetic and
invariants that follow from the definition.

Source: "量化" tutorial (aiknowledge.cn), "量化怎么工作": asymmetric
quantization adds a zero point to the rounded quotient, for distributions not
centred on zero (its example: non-negative ReLU outputs, where a symmetric
range wastes half of the codes).  Readings (stated in the oracle): the range
is widened to hold 0; L = 2^b - 1 codes above 0; s = fl32(range / L);
z = rint(-lo / s); codes rint(w / s) + z clipped to [0, L]."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload

SRC = os.path.join(os.path.dirname(oracle.__file__), "dq_oracle.c")


def f32(v):
    return np.float32(v)


def check_nonnegative_rows(orc) -> list[str]:
    """A non-negative row (the page's ReLU case) needs no negative codes: the
    zero point is 0, the largest element takes the top code L, the zeros code
    0, and every code is the nearest integer to fl32(w / s) (ties to even)."""
    bad = []
    rng = np.random.default_rng(21)
    for bits in (2, 4, 5, 8, 11, 15):
        L = (1 << bits) - 1
        w = np.abs(rng.standard_normal((3, 37))).astype(np.float32)
        w[:, 5] = 0.0
        packed, s, z, u = orc.quantize_pack_asym(w, bits)
        for n in range(3):
            if z[n] != 0:
                bad.append("b=%d nonneg row %d: zero point %d" % (bits, n, z[n]))
            if u[n, int(np.argmax(w[n]))] != L or u[n, 5] != 0:
                bad.append("b=%d nonneg row %d: max/zero codes" % (bits, n))
            # the scale: fl32(max / L), as an exact rational rounded once
            want_s = f32(float(Fraction(float(w[n].max())) / L))
            if s[n] != want_s and abs(Fraction(float(s[n])) - Fraction(float(w[n].max())) / L) > \
                    abs(Fraction(float(want_s)) - Fraction(float(w[n].max())) / L):
                bad.append("b=%d nonneg row %d: scale %r" % (bits, n, s[n]))
            for k in range(37):
                t = Fraction(float(f32(w[n, k]) / s[n]))
                c = int(u[n, k])
                d = abs(t - c)
                if d > Fraction(1, 2) or (d == Fraction(1, 2) and c % 2):
                    bad.append("b=%d nonneg code %d,%d" % (bits, n, k))
                    break
        # exact ties: the top element L * 2^-6 makes s = 2^-6 exactly, so
        # (j + 1/2) * 2^-6 sits halfway between codes j and j + 1: the even one
        s0 = 2.0 ** -6
        js = np.arange(min(L, 40))
        row = np.concatenate([[L * s0], (js + 0.5) * s0]).astype(np.float32)[None, :]
        _, s1, z1, u1 = orc.quantize_pack_asym(row, bits)
        want = np.where(js % 2 == 0, js, js + 1)
        if s1[0] != f32(s0) or z1[0] != 0 or not np.array_equal(u1[0, 1:], want):
            bad.append("b=%d ties" % bits)
    return bad


def check_nonpositive_rows(orc) -> list[str]:
    """A non-positive row: the zero point is L and the smallest element gets
    code 0 (-lo / s lies within L * 2^-24 of L)."""
    bad = []
    rng = np.random.default_rng(22)
    for bits in (3, 6, 9, 14):
        L = (1 << bits) - 1
        w = -np.abs(rng.standard_normal((2, 29))).astype(np.float32)
        _, s, z, u = orc.quantize_pack_asym(w, bits)
        for n in range(2):
            if z[n] != L or u[n, int(np.argmin(w[n]))] != 0:
                bad.append("b=%d nonpos row %d: z=%d" % (bits, n, z[n]))
    return bad


def f32_nearest(q: Fraction) -> float:
    """The fp32 value nearest to the rational q, ties to the even significand
    (IEEE round to nearest; subnormals kept, overflow to infinity), computed
    with exact integers only."""
    if q == 0:
        return 0.0
    sign, a = (-1.0 if q < 0 else 1.0), abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)  # 24 significant bits, or the subnormal step
    m = a / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    if v >= Fraction(2) ** 128 - Fraction(2) ** 103:
        return sign * float("inf")
    return sign * float(v)  # exact: v has at most 24 significant bits


def rint_even(q: Fraction) -> int:
    n = q.numerator // q.denominator
    r = q - n
    return n + 1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1)) else n


def check_mixed_sign_scale(orc) -> list[str]:
    """Rows with both signs (reading of "量化怎么工作" taken by the oracle: the
    range [lo, hi] is widened to hold 0, s = fl32(fl32(hi - lo) / L) with both
    operations rounded in fp32, z = clip(rint(fl32(-lo / s)), 0, L)).  The
    expected s and z come from exact rationals rounded by f32_nearest, so a
    range formed in fp64, a divide split as hi/L - lo/L, or a zero point from
    an unrounded quotient disagree on some rows.  Invariants: the smallest
    element gets code 0 (rint(lo/s) + rint(-lo/s) = 0, rint being odd), the
    largest code L - 1 or L."""
    bad = []
    rng = np.random.default_rng(23)
    for bits in range(2, 16):
        L = (1 << bits) - 1
        # mixed-sign rows of varied skew and magnitude: N(mu, 1) * 2^e
        mu = rng.uniform(-1.5, 1.5, 40)
        ex = rng.integers(-20, 20, 40).astype(np.float64)
        w = ((rng.standard_normal((40, 33)) + mu[:, None]) * 2.0 ** ex[:, None]).astype(np.float32)
        w[:, 0] = -np.abs(w[:, 0]) - np.float32(2.0 ** ex[0] * 1e-3)  # a negative element
        w[:, 1] = np.abs(w[:, 1]) + np.float32(2.0 ** ex[0] * 1e-3)   # and a positive one
        _, s, z, u = orc.quantize_pack_asym(w, bits)
        for n in range(40):
            lo, hi = Fraction(float(w[n].min())), Fraction(float(w[n].max()))
            want_s = f32_nearest(Fraction(f32_nearest(hi - lo)) / L)
            if np.float32(s[n]).view(np.uint32) != np.float32(want_s).view(np.uint32):
                bad.append("b=%d mixed row %d: scale %r, want %r" % (bits, n, s[n], want_s))
                continue
            want_z = min(max(rint_even(Fraction(f32_nearest(-lo / Fraction(want_s)))), 0), L)
            if z[n] != want_z:
                bad.append("b=%d mixed row %d: zero point %d, want %d" % (bits, n, z[n], want_z))
            if u[n, int(np.argmin(w[n]))] != 0 or u[n, int(np.argmax(w[n]))] < L - 1:
                bad.append("b=%d mixed row %d: extreme codes" % (bits, n))
    return bad


def check_error_bound(orc) -> list[str]:
    """|w - (u - z) s| <= s (1 + 2^-20): half a step from rounding w / s and half
    a step from rounding the zero point, plus the fp32 roundings."""
    bad = []
    for bits in range(2, 16):
        w = workload.weights(97, bits, 8, 300, dtype="f32")
        w[1] += np.float32(0.05)  # shifted rows: the zero point moves
        w[2] = np.abs(w[2])
        packed, s, z, u = orc.quantize_pack_asym(w, bits)
        for n in range(8):
            err = np.abs(w[n].astype(np.float64) - (u[n].astype(np.float64) - z[n]) * float(s[n]))
            if err.max() > float(s[n]) * (1 + 2 ** -20):
                bad.append("b=%d row %d error %g > s %g" % (bits, n, err.max(), s[n]))
            if u[n].max() >= (1 << bits) or z[n] < 0 or z[n] >= (1 << bits):
                bad.append("b=%d row %d out of range" % (bits, n))
    return bad


def check_special_rows(orc) -> list[str]:
    bad = []
    for bits in (2, 7, 15):
        L = (1 << bits) - 1
        half = 1 << (bits - 1)
        w = np.zeros((4, 5), np.float32)
        w[1, 2] = np.nan
        w[2] = [3e38, -1e38, 0, 1, 2]          # range overflows fp32
        w[3] = [1.4e-45, 0, 0, 0, 0]            # one subnormal step: range / L underflows
        _, s, z, u = orc.quantize_pack_asym(w, bits)
        if not (s[0] == f32(1.0) / f32(L) and z[0] == 0 and not u[0].any()):
            bad.append("b=%d zero row" % bits)
        for n in (1, 2):
            if not (np.isnan(s[n]) and z[n] == half and (u[n] == half).all()):
                bad.append("b=%d non-finite row %d" % (bits, n))
        if not (s[3] == f32(1.0) / f32(L) and z[3] == 0 and not u[3].any()):
            bad.append("b=%d underflow row" % bits)
    return bad


def check_unpack_and_matmul(orc) -> list[str]:
    """Unpack gives u - z and fl32((u - z) s); the fp64 product equals the exact
    rational s * sum x (u - z) (N, K small), and a one-hot x picks one weight."""
    bad = []
    for bits in (2, 5, 8, 12, 15):
        w = workload.weights(98, bits, 5, 7, dtype="f32")
        w[0] = np.abs(w[0])
        packed, s, z, u = orc.quantize_pack_asym(w, bits)
        q, w_hat = orc.unpack_asym(packed, s, z, 5, 7, bits)
        if not np.array_equal(q, u.astype(np.int64) - z[:, None]):
            bad.append("b=%d unpack codes" % bits)
        if not np.array_equal(w_hat, q.astype(np.float32) * s[:, None]):
            bad.append("b=%d unpack dequant" % bits)
        x = workload.activations(98, bits, 3, 7)
        xf = workload.bf16_to_f32(x)
        y, bound = orc.matmul_asym(x, packed, s, z, 5, 7, bits)
        for m in range(3):
            for n in range(5):
                acc = sum(Fraction(float(xf[m, k])) * (int(u[n, k]) - int(z[n])) for k in range(7))
                mag = sum(abs(Fraction(float(xf[m, k])) * (int(u[n, k]) - int(z[n]))) for k in range(7))
                if y[m, n] != float(Fraction(float(s[n])) * acc) or \
                        bound[m, n] != float(abs(Fraction(float(s[n]))) * mag):
                    bad.append("b=%d matmul (%d,%d)" % (bits, m, n))
        onehot = np.zeros((1, 7), np.uint16)
        onehot[0, 3] = 0x3F80  # 1.0
        y, _ = orc.matmul_asym(onehot, packed, s, z, 5, 7, bits)
        if not np.array_equal(y[0].astype(np.float32), w_hat[:, 3]):
            bad.append("b=%d one-hot" % bits)
    return bad


CHECKS = [check_nonnegative_rows, check_nonpositive_rows, check_mixed_sign_scale,
          check_error_bound, check_special_rows, check_unpack_and_matmul]


def run_all(orc) -> list[str]:
    bad = []
    for c in CHECKS:
        bad += c(orc)
    return bad


@pytest.mark.parametrize("check", CHECKS)
def test_asym_oracle_pinned(check):
    assert check(oracle.default()) == []


MUTANTS = [
    ("levels_minus_one", "const int32_t L = (1 << bits) - 1;", "const int32_t L = (1 << bits) - 2;"),
    ("range_without_zero", "float lo = 0.0f, hi = 0.0f;\n    int nonfinite = 0;\n    for (int64_t k = 0; k < K; k++) {\n        float v = load_weight(w, dtype, row * K + k);\n        if (!isfinite(v))\n            nonfinite = 1;",
     "float lo = 1e30f, hi = -1e30f;\n    int nonfinite = 0;\n    for (int64_t k = 0; k < K; k++) {\n        float v = load_weight(w, dtype, row * K + k);\n        if (!isfinite(v))\n            nonfinite = 1;"),
    ("range_in_fp64", "float s = (range == 0.0f ? 1.0f : range) / (float)L;",
     "float s = range == 0.0f ? 1.0f / (float)L : (float)(((double)hi - (double)lo) / (double)L);"),
    ("scale_divide_split", "float s = (range == 0.0f ? 1.0f : range) / (float)L;",
     "float s = range == 0.0f ? 1.0f / (float)L : hi / (float)L - lo / (float)L;"),
    ("zero_point_truncated", "float zf = rintf(-lo / s);", "float zf = truncf(-lo / s);"),
    ("zero_point_subtracted", "float c = rintf(quot) + zf;", "float c = rintf(quot) - zf;"),
    ("codes_round_half_up", "float c = rintf(quot) + zf;", "float c = roundf(quot) + zf;"),
    ("nonfinite_zero_point_0", "*zero = (int32_t)half;", "*zero = 0;"),
    ("unpack_adds_zero", "int32_t q = (int32_t)u[k] - zeros[n];", "int32_t q = (int32_t)u[k] + zeros[n];"),
    ("matmul_ignores_zero", "(double)((int32_t)u[k] - zeros[n]);", "(double)((int32_t)u[k]);"),
    ("unsigned_pack_msb_first", "words[pos / 32] |= ((u[k] >> j) & 1u) << (pos % 32);",
     "words[pos / 32] |= ((u[k] >> (bits - 1 - j)) & 1u) << (pos % 32);"),
]


def test_asym_pins_accept_the_oracle():
    assert run_all(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_asym_pins_reject_mutant(tmp_path, name, old, new):
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


def test_f32_nearest_is_ieee_rounding():
    """The rounding helper of the mixed-sign pin agrees with the IEEE fp64 ->
    fp32 conversion (one correct rounding of an exact double) on normal,
    subnormal, tie and overflowing values."""
    rng = np.random.default_rng(5)
    d = np.concatenate([rng.standard_normal(2000) * 2.0 ** rng.integers(-160, 130, 2000),
                        (rng.integers(1, 1 << 24, 200) + 0.5) * 2.0 ** -20,  # ties
                        [1.5 * 2.0 ** -149, 2.0 ** -150, 3.4e38, 3.403e38, -7e-46, 1e-300]])
    with np.errstate(over="ignore"):
        want = d.astype(np.float32)
    for v, wv in zip(d, want):
        assert np.float32(f32_nearest(Fraction(float(v)))).view(np.uint32) == wv.view(np.uint32), v
