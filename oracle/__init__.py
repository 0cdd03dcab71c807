"""CPU oracle for per-row symmetric b-bit quantization, bit packing and the
dequantized matmul.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
package never imports it and shares no code with it.

The arithmetic lives in ``dq_oracle.c`` (plain C, built with gcc, no fast-math,
no FMA contraction).  This module only marshals numpy arrays.  Each function
names the passage it follows:

* quantizer -- "量化" tutorial (aiknowledge.cn), "how quantization works" and
  "Step 1" symmetric per-channel code, one channel = one row of W[N, K];
* packing -- DynaQuant page (zingnex.cn), "custom kernel architecture" (packed
  N-bit storage) and "status and roadmap" (pack / unpack utilities);
* matmul -- BPDQ article (devpress.csdn.net) section 3.2 (dequantize fused
  with the product, fp32 scales, fp32 output), computed here in fp64;
* asymmetric variant -- "量化" tutorial, "how quantization works" (a zero
  point added to the rounded quotient for distributions not centred on zero):
  per-row scale and zero point, unsigned codes;
* group-wise scales -- "量化" tutorial, exercise 1 of its exercises section (one
  scale per group of g weights instead of per channel).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdq_oracle.so")

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-Wall", "-Wextra", "-shared", "-fPIC"]

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``src`` (default: the oracle) with gcc into the shared library ``out``."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp])
        os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_bits(bits: int):
    if not 2 <= bits <= 15:
        raise ValueError("bits must be in [2, 15]")


class Oracle:
    """numpy marshalling around one build of ``dq_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.oracle_row_bytes.argtypes = [i64, i32]
        lib.oracle_row_bytes.restype = i64
        lib.oracle_quantize_pack.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp]
        lib.oracle_quantize_pack.restype = None
        lib.oracle_pack.argtypes = [vp, i64, i64, i32, vp]
        lib.oracle_pack.restype = None
        lib.oracle_unpack.argtypes = [vp, vp, i64, i64, i32, vp, vp]
        lib.oracle_unpack.restype = None
        lib.oracle_matmul.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp, vp]
        lib.oracle_matmul.restype = None
        lib.oracle_matmul_pairs.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp, vp, i64, vp, vp]
        lib.oracle_matmul_pairs.restype = None
        lib.oracle_quantize_pack_asym.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp]
        lib.oracle_quantize_pack_asym.restype = None
        lib.oracle_unpack_asym.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp]
        lib.oracle_unpack_asym.restype = None
        lib.oracle_matmul_asym.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, vp, vp]
        lib.oracle_matmul_asym.restype = None
        lib.oracle_quantize_pack_group.argtypes = [vp, i32, i64, i64, i32, i64, vp, vp, vp]
        lib.oracle_quantize_pack_group.restype = None
        lib.oracle_unpack_group.argtypes = [vp, vp, i64, i64, i32, i64, vp, vp]
        lib.oracle_unpack_group.restype = None
        lib.oracle_matmul_group.argtypes = [vp, i64, vp, vp, i64, i64, i32, i64, vp, vp]
        lib.oracle_matmul_group.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        """Thread count of the OpenMP loops from now on (for timing)."""
        self.lib.oracle_set_threads(int(n))

    def row_bytes(self, K: int, bits: int) -> int:
        """Bytes of one packed row: ceil(K*bits/8) rounded up to a multiple of 128."""
        return int(self.lib.oracle_row_bytes(K, bits))

    def quantize_pack(self, w: np.ndarray, bits: int):
        """Quantize W[N, K] per row and pack it.

        ``w`` is float32, or uint16 holding bf16 bit patterns.
        Returns (packed uint32 [N, row_bytes/4], scales float32 [N], q int32 [N, K]).
        """
        _check_bits(bits)
        w = np.ascontiguousarray(w)
        if w.dtype == np.float32:
            dtype = 0
        elif w.dtype == np.uint16:
            dtype = 1
        else:
            raise TypeError("w must be float32 or uint16 (bf16 bits)")
        N, K = w.shape
        packed = np.empty((N, self.row_bytes(K, bits) // 4), dtype=np.uint32)
        scales = np.empty((N,), dtype=np.float32)
        q = np.empty((N, K), dtype=np.int32)
        self.lib.oracle_quantize_pack(_ptr(w), dtype, N, K, bits, _ptr(packed), _ptr(scales), _ptr(q))
        return packed, scales, q

    def pack(self, q: np.ndarray, bits: int) -> np.ndarray:
        """Pack int32 codes q[N, K] (each in [-2^(b-1), 2^(b-1))) into [N, row_bytes/4] words."""
        _check_bits(bits)
        q = np.ascontiguousarray(q, dtype=np.int32)
        N, K = q.shape
        lim = 1 << (bits - 1)
        if q.size and (q.min() < -lim or q.max() >= lim):
            raise ValueError("code out of range for %d bits" % bits)
        packed = np.empty((N, self.row_bytes(K, bits) // 4), dtype=np.uint32)
        self.lib.oracle_pack(_ptr(q), N, K, bits, _ptr(packed))
        return packed

    def unpack(self, packed: np.ndarray, scales, N: int, K: int, bits: int):
        """Inverse of the packing.  Returns (q int32 [N, K], w_hat float32 [N, K] or None)."""
        _check_bits(bits)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        assert packed.size == N * (self.row_bytes(K, bits) // 4)
        q = np.empty((N, K), dtype=np.int32)
        w_hat = None
        if scales is not None:
            scales = np.ascontiguousarray(scales, dtype=np.float32)
            w_hat = np.empty((N, K), dtype=np.float32)
        self.lib.oracle_unpack(_ptr(packed), _ptr(scales), N, K, bits, _ptr(q), _ptr(w_hat))
        return q, w_hat

    def matmul(self, x_bf16: np.ndarray, packed: np.ndarray, scales: np.ndarray, N: int, K: int,
               bits: int):
        """fp64 y[M, N] = s[n] * sum_k x[m,k] q[n,k] and bound[M, N] = |s| * sum_k |x q|."""
        _check_bits(bits)
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M = x.shape[0]
        assert x.shape == (M, K)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        y = np.empty((M, N), dtype=np.float64)
        bound = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_matmul(_ptr(x), M, _ptr(packed), _ptr(scales), N, K, bits, _ptr(y),
                               _ptr(bound))
        return y, bound

    def matmul_pairs(self, x_bf16: np.ndarray, packed: np.ndarray, scales: np.ndarray, N: int,
                     K: int, bits: int, ms, ns):
        """``matmul`` for the listed (m, n) pairs only.  Returns (y, bound) 1-D fp64."""
        _check_bits(bits)
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M = x.shape[0]
        assert x.shape == (M, K)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        assert ms.shape == ns.shape
        assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        y = np.empty(ms.shape, dtype=np.float64)
        bound = np.empty(ms.shape, dtype=np.float64)
        self.lib.oracle_matmul_pairs(_ptr(x), M, _ptr(packed), _ptr(scales), N, K, bits,
                                     _ptr(ms), _ptr(ns), ms.size, _ptr(y), _ptr(bound))
        return y, bound


    # -- asymmetric variant ([TUT] "how quantization works": zero point)

    def quantize_pack_asym(self, w: np.ndarray, bits: int):
        """Per-row scale and zero point.  Returns (packed uint32 [N, row_bytes/4],
        scales float32 [N], zeros int32 [N], codes uint32 [N, K])."""
        _check_bits(bits)
        w = np.ascontiguousarray(w)
        dtype = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1}.get(w.dtype)
        if dtype is None:
            raise TypeError("w must be float32 or uint16 (bf16 bits)")
        N, K = w.shape
        packed = np.empty((N, self.row_bytes(K, bits) // 4), dtype=np.uint32)
        scales = np.empty((N,), dtype=np.float32)
        zeros = np.empty((N,), dtype=np.int32)
        u = np.empty((N, K), dtype=np.uint32)
        self.lib.oracle_quantize_pack_asym(_ptr(w), dtype, N, K, bits, _ptr(packed), _ptr(scales),
                                           _ptr(zeros), _ptr(u))
        return packed, scales, zeros, u

    def unpack_asym(self, packed, scales, zeros, N: int, K: int, bits: int):
        """(q = u - z int32 [N, K], w_hat = fl32(q * s) float32 [N, K])."""
        _check_bits(bits)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        zeros = np.ascontiguousarray(zeros, dtype=np.int32)
        q = np.empty((N, K), dtype=np.int32)
        w_hat = np.empty((N, K), dtype=np.float32)
        self.lib.oracle_unpack_asym(_ptr(packed), _ptr(scales), _ptr(zeros), N, K, bits, _ptr(q),
                                    _ptr(w_hat))
        return q, w_hat

    def matmul_asym(self, x_bf16, packed, scales, zeros, N: int, K: int, bits: int):
        """fp64 y = s * sum x (u - z) and bound = |s| * sum |x (u - z)|, [M, N]."""
        _check_bits(bits)
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M = x.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        bound = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_matmul_asym(_ptr(x), M, _ptr(np.ascontiguousarray(packed, dtype=np.uint32)),
                                    _ptr(np.ascontiguousarray(scales, dtype=np.float32)),
                                    _ptr(np.ascontiguousarray(zeros, dtype=np.int32)), N, K, bits,
                                    _ptr(y), _ptr(bound))
        return y, bound


    # -- group-wise scales ([TUT] exercise: one scale per g weights of a row)

    def quantize_pack_group(self, w: np.ndarray, bits: int, g: int):
        """Returns (packed, scales float32 [N, ceil(K/g)], q int32 [N, K])."""
        _check_bits(bits)
        w = np.ascontiguousarray(w)
        dtype = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1}.get(w.dtype)
        if dtype is None:
            raise TypeError("w must be float32 or uint16 (bf16 bits)")
        N, K = w.shape
        G = -(-K // g)
        packed = np.empty((N, self.row_bytes(K, bits) // 4), dtype=np.uint32)
        scales = np.empty((N, G), dtype=np.float32)
        q = np.empty((N, K), dtype=np.int32)
        self.lib.oracle_quantize_pack_group(_ptr(w), dtype, N, K, bits, g, _ptr(packed),
                                            _ptr(scales), _ptr(q))
        return packed, scales, q

    def unpack_group(self, packed, scales, N: int, K: int, bits: int, g: int):
        _check_bits(bits)
        q = np.empty((N, K), dtype=np.int32)
        w_hat = np.empty((N, K), dtype=np.float32)
        self.lib.oracle_unpack_group(_ptr(np.ascontiguousarray(packed, dtype=np.uint32)),
                                     _ptr(np.ascontiguousarray(scales, dtype=np.float32)), N, K,
                                     bits, g, _ptr(q), _ptr(w_hat))
        return q, w_hat

    def matmul_group(self, x_bf16, packed, scales, N: int, K: int, bits: int, g: int):
        """fp64 y = sum_k x q s[n, k/g] and bound = sum_k |x q s[n, k/g]|, [M, N]."""
        _check_bits(bits)
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M = x.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        bound = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_matmul_group(_ptr(x), M, _ptr(np.ascontiguousarray(packed, dtype=np.uint32)),
                                     _ptr(np.ascontiguousarray(scales, dtype=np.float32)), N, K,
                                     bits, g, _ptr(y), _ptr(bound))
        return y, bound


def default() -> Oracle:
    """The oracle built from ``dq_oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _default = Oracle(_LIB_PATH)
    return _default


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def row_bytes(K: int, bits: int) -> int:
    return default().row_bytes(K, bits)


def quantize_pack(w: np.ndarray, bits: int):
    return default().quantize_pack(w, bits)


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    return default().pack(q, bits)


def unpack(packed: np.ndarray, scales, N: int, K: int, bits: int):
    return default().unpack(packed, scales, N, K, bits)


def matmul(x_bf16, packed, scales, N: int, K: int, bits: int):
    return default().matmul(x_bf16, packed, scales, N, K, bits)


def matmul_pairs(x_bf16, packed, scales, N: int, K: int, bits: int, ms, ns):
    return default().matmul_pairs(x_bf16, packed, scales, N, K, bits, ms, ns)


def quantize_pack_asym(w: np.ndarray, bits: int):
    return default().quantize_pack_asym(w, bits)


def unpack_asym(packed, scales, zeros, N: int, K: int, bits: int):
    return default().unpack_asym(packed, scales, zeros, N, K, bits)


def matmul_asym(x_bf16, packed, scales, zeros, N: int, K: int, bits: int):
    return default().matmul_asym(x_bf16, packed, scales, zeros, N, K, bits)


def quantize_pack_group(w: np.ndarray, bits: int, g: int):
    return default().quantize_pack_group(w, bits, g)


def unpack_group(packed, scales, N: int, K: int, bits: int, g: int):
    return default().unpack_group(packed, scales, N, K, bits, g)


def matmul_group(x_bf16, packed, scales, N: int, K: int, bits: int, g: int):
    return default().matmul_group(x_bf16, packed, scales, N, K, bits, g)
