"""Independent checks that pin the CPU oracle to what the pages and the
mathematics fix.  None of them re-runs the oracle's own arithmetic: they use
exact rational arithmetic (fractions), brute-force search over the integer
levels, Python big-integer bit streams and closed forms.

Sources: "量化" (Quantization) tutorial, aiknowledge.cn, "how quantization
works" / "Step 1" (symmetric per-channel quantizer, error at most scale/2);
DynaQuant page, zingnex.cn, "custom kernel architecture" (packed N-bit
storage); BPDQ article section 3.2 (dequantize fused into the matmul).

Each ``check_*`` returns a list of human-readable violations (empty = pass) so
that the mutation tests can assert that a planted mistake is caught.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32_QNAN_BITS = 0x7FC00000


def f32_bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


def f32_round(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to an even significand.
    Decided by exact comparison of the neighbouring candidates."""
    c = np.float32(float(fr))
    lo = np.nextafter(c, np.float32(-np.inf))
    hi = np.nextafter(c, np.float32(np.inf))
    best = None
    for cand in (lo, c, hi):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - fr)
        key = (d, f32_bits(cand) & 1)  # on a tie prefer the even bit pattern
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def nearest_level(t: Fraction, lo: int, hi: int) -> int:
    """The integer in [lo, hi] nearest to t, ties to the even one, by exhaustive
    comparison.  |t - j| is convex in j, so besides the two ends only the
    integers next to t can win; those are the candidates compared."""
    import math
    cands = {lo, hi}
    for j in range(math.floor(t) - 1, math.ceil(t) + 2):
        if lo <= j <= hi:
            cands.add(j)
    best = None
    for j in sorted(cands):
        key = (abs(t - j), j & 1)
        if best is None or key < best[0]:
            best = (key, j)
    return best[1]


def check_quantize_row(w: np.ndarray, bits: int, q: np.ndarray, s) -> list[str]:
    """Exact check of one row: scale and every code, by rational arithmetic and
    brute force over the 2^b levels.  ``w`` fp32 values, ``q`` int codes, ``s`` fp32."""
    bad = []
    w = np.asarray(w, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    if not np.all(np.isfinite(w)):
        if f32_bits(s) != F32_QNAN_BITS:
            bad.append("non-finite row: scale bits %08x, want 7fc00000" % f32_bits(s))
        if np.any(np.asarray(q) != 0):
            bad.append("non-finite row: codes not all 0")
        return bad
    a = max((abs(Fraction(float(v))) for v in w), default=Fraction(0))
    want_s = f32_round((a if a != 0 else Fraction(1)) / qmax)
    zero_row = a == 0 or want_s == 0
    if want_s == 0:
        want_s = f32_round(Fraction(1, qmax))
    if f32_bits(s) != f32_bits(want_s):
        bad.append("scale %r (bits %08x), want %r (bits %08x)" % (
            float(s), f32_bits(s), float(want_s), f32_bits(want_s)))
        return bad
    sf = Fraction(float(want_s))
    for k, v in enumerate(w):
        if zero_row:
            want = 0
        else:
            t = Fraction(float(f32_round(Fraction(float(v)) / sf)))
            want = nearest_level(t, -qmax - 1, qmax)
        if int(q[k]) != want:
            bad.append("k=%d w=%r: q=%d, want %d" % (k, float(v), int(q[k]), want))
    return bad


def check_quantize_invariants(w: np.ndarray, bits: int, q: np.ndarray, s: np.ndarray) -> list[str]:
    """Vectorised invariants for larger finite matrices (one scale per row):
    the absmax element maps to +-qmax, |fl32(w/s) - q| <= 1/2, code 0 (q = -qmax-1)
    never occurs when s is a normal number, and |w - q s| <= s (1/2 + (qmax+1) 2^-24)
    (the tutorial's scale/2 bound, widened by the fp32 rounding of w/s)."""
    bad = []
    w = np.asarray(w, dtype=np.float32)
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    a = np.max(np.abs(w), axis=1)
    nz = a > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = w / s[:, None]  # IEEE fp32 divide
    rows = np.nonzero(nz)[0]
    if rows.size:
        arg = np.argmax(np.abs(w[rows]), axis=1)
        qa = q[rows, arg]
        if not np.all(np.abs(qa) == qmax):
            bad.append("absmax element not mapped to +-qmax in %d rows" % int(np.sum(np.abs(qa) != qmax)))
        d = np.abs(t[rows] - q[rows])
        if not np.all(d <= 0.5):
            bad.append("|t - q| > 1/2 at %d elements" % int(np.sum(d > 0.5)))
        normal = s[rows] >= np.finfo(np.float32).tiny
        if np.any(q[rows][normal] == -qmax - 1):
            bad.append("code 0 (q = -qmax-1) used")
        err = np.abs(w[rows].astype(np.float64) - q[rows] * s[rows, None].astype(np.float64))
        lim = s[rows, None].astype(np.float64) * (0.5 + (qmax + 1) * 2.0 ** -24)
        if not np.all(err <= lim):
            bad.append("|w - q s| beyond s(1/2 + (qmax+1)2^-24) at %d elements" % int(np.sum(err > lim)))
    if np.any(q[~nz] != 0):
        bad.append("zero row with non-zero codes")
    return bad


def row_bytes_formula(K: int, bits: int) -> int:
    return -(-(-(-K * bits // 8)) // 128) * 128


def stream_words(q_row: np.ndarray, bits: int, row_words: int) -> list[int]:
    """The packed row built as one Python integer: code k = q + 2^(b-1) shifted to bit k*b."""
    stream = 0
    for k, v in enumerate(q_row):
        stream |= (int(v) + (1 << (bits - 1))) << (k * bits)
    return [(stream >> (32 * i)) & 0xFFFFFFFF for i in range(row_words)]


def check_pack(q: np.ndarray, bits: int, packed: np.ndarray) -> list[str]:
    bad = []
    N, K = q.shape
    rw = row_bytes_formula(K, bits) // 4
    if packed.shape != (N, rw):
        return ["packed shape %s, want %s" % (packed.shape, (N, rw))]
    for n in range(N):
        want = stream_words(q[n], bits, rw)
        got = [int(v) for v in packed[n]]
        if got != want:
            i = next(i for i in range(rw) if got[i] != want[i])
            bad.append("row %d word %d: %08x, want %08x" % (n, i, got[i], want[i]))
    return bad


def check_matmul_exact(x_f32: np.ndarray, q: np.ndarray, s: np.ndarray, y: np.ndarray,
                       bound: np.ndarray, rel: float = 1e-12) -> list[str]:
    """Exact rational y = s[n] * sum_k x[m,k] q[n,k] and B = |s| sum |x q| on tiny shapes."""
    bad = []
    M, K = x_f32.shape
    N = q.shape[0]
    for m in range(M):
        for n in range(N):
            sf = Fraction(float(s[n]))
            terms = [Fraction(float(x_f32[m, k])) * int(q[n, k]) for k in range(K)]
            ye = sf * sum(terms, Fraction(0))
            be = abs(sf) * sum((abs(t) for t in terms), Fraction(0))
            tol = rel * float(be) + 1e-300
            if abs(float(ye) - y[m, n]) > tol:
                bad.append("y[%d,%d]=%r, exact %r" % (m, n, y[m, n], float(ye)))
            if abs(float(be) - bound[m, n]) > tol:
                bad.append("bound[%d,%d]=%r, exact %r" % (m, n, bound[m, n], float(be)))
    return bad


def within_tolerance(y_test: np.ndarray, y_ref: np.ndarray, bound: np.ndarray,
                     rel: float = 1e-4) -> np.ndarray:
    """|y - y_ref| <= rel * B, and y exactly zero where B == 0."""
    y_test = np.asarray(y_test, dtype=np.float64)
    ok = np.abs(y_test - y_ref) <= rel * bound
    zero = bound == 0
    ok[zero] = y_test[zero] == 0
    return ok
