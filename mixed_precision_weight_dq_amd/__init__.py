"""Python binding of ``libdq.so``: packed b-bit weight quantization and the
dequantized GEMV / GEMM on MI355X (gfx950).

Two layers, both argument marshalling only (every step runs in the HIP
kernels behind the C ABI declared in ``include/dq.h``):

* ``dq_packed_row_bytes``, ``dq_quantize_pack``, ``dq_row_sumsq``,
  ``dq_quantize_pack_sumsq``, ``dq_unpack``, ``dq_gemv``, ``dq_gemv_batched``, ``dq_gemm``,
  ``dq_stream_read``,
  ``dq_sensitivity``, ``dq_allocate_bits`` -- the C entry points under their
  own names, taking integer addresses (device memory, host memory for the last
  two) and sizes; they return the ``dq_status`` code.
* ``quantize_pack``, ``row_sumsq``, ``quantize_pack_sumsq``, ``unpack``, ``gemv``,
  ``gemv_batched``, ``gemm``, ``stream_read`` -- the same calls on torch tensors (torch provides device
  memory and the current stream); they check device, dtype and contiguity,
  allocate outputs with torch and raise ``DQError`` on a non-zero status.
* ``quantize_pack_asym``, ``unpack_asym``, ``gemv_asym``, ``gemm_asym`` --
  the asymmetric (zero-point) variant on torch tensors.
* ``quantize_pack_group``, ``unpack_group``, ``gemv_group``, ``gemm_group``
  -- group-wise scales (one per g codes of a row) on torch tensors.
* ``sensitivity``, ``allocate_bits`` -- the host-side allocation calls on
  numpy arrays (the recipe: one bit width per matrix).
* ``write_packed_file``, ``PackedFile`` -- the on-disk packed-weight format
  (``dq_file_*``): write a recipe's packed matrices from host arrays, map a
  file, read its entries as numpy views and copy them into GPU tensors.

``dq_stream_read`` is not a step of the method: a plain streaming read that
measures what a kernel bound by HBM reaches at a given size.

There is no fallback: if the library is missing or the device is not a GPU,
the calls fail.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "DQError", "DQ_F32", "DQ_BF16", "library_path", "dq_packed_row_bytes", "dq_quantize_pack",
    "dq_unpack", "dq_gemv", "dq_gemm", "dq_stream_read", "dq_status_string", "dq_last_error",
    "packed_row_bytes", "quantize_pack", "unpack", "gemv", "gemm", "stream_read", "load",
    "dq_row_sumsq", "row_sumsq", "dq_quantize_pack_sumsq", "dq_sensitivity", "dq_allocate_bits", "quantize_pack_sumsq",
    "sensitivity", "allocate_bits", "NATIVE_LEVELS", "FULL_LEVELS", "DQFileMatrix",
    "write_packed_file", "PackedFile", "dq_quantize_pack_asym", "dq_unpack_asym",
    "dq_gemv_asym", "dq_gemm_asym", "quantize_pack_asym", "unpack_asym", "gemv_asym",
    "gemm_asym", "dq_quantize_pack_group", "dq_unpack_group", "dq_gemv_group", "dq_gemm_group",
    "quantize_pack_group", "unpack_group", "gemv_group", "gemm_group", "DQGemvItem",
    "GEMV_BATCH_MAX", "dq_gemv_batched", "gemv_batched",
]

(DQ_OK, DQ_ERR_NULL, DQ_ERR_BITS, DQ_ERR_SHAPE, DQ_ERR_ALIGN, DQ_ERR_DTYPE, DQ_ERR_HIP,
 DQ_ERR_BUDGET, DQ_ERR_VALUE, DQ_ERR_IO, DQ_ERR_FORMAT) = range(11)
DQ_F32, DQ_BF16 = 0, 1
GEMV_MAX_M = 16
NATIVE_LEVELS = (4, 8, 16)        # hardware-native allocation levels (16 = BF16 kept)
FULL_LEVELS = tuple(range(4, 17))  # every width from 4 to 16

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdq.so")
_lib = None


class DQFileMatrix(ctypes.Structure):
    """``dq_file_matrix`` of include/dq.h."""
    _fields_ = [("name", ctypes.c_char * 64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class DQGemvItem(ctypes.Structure):
    """``dq_gemv_item`` of include/dq.h (device addresses and sizes)."""
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("zeros", ctypes.c_void_p)]


GEMV_BATCH_MAX = 32


class DQError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = "%s: %s" % (where, dq_status_string(status))
        if status == DQ_ERR_HIP:
            msg += " (%s)" % dq_last_error()
        super().__init__(msg)
        self.status = status


def load():
    """Load libdq.so (built in-tree by ``mixed_precision_weight_dq_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError("libdq.so is not built (%s); run __graft_entry__.build() or "
                          "python -m mixed_precision_weight_dq_amd.build" % library_path)
    lib = ctypes.CDLL(library_path)
    i64, i32, vp, st = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32
    lib.dq_packed_row_bytes.argtypes = [i64, i32]
    lib.dq_packed_row_bytes.restype = ctypes.c_size_t
    lib.dq_quantize_pack.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp]
    lib.dq_quantize_pack.restype = st
    lib.dq_unpack.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
    lib.dq_unpack.restype = st
    lib.dq_gemv.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp, vp]
    lib.dq_gemv.restype = st
    lib.dq_gemm.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp, vp]
    lib.dq_gemm.restype = st
    lib.dq_gemv_batched.argtypes = [vp, i32, i64, vp]
    lib.dq_gemv_batched.restype = st
    lib.dq_stream_read.argtypes = [vp, i64, vp, i64, vp]
    lib.dq_stream_read.restype = st
    lib.dq_row_sumsq.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    lib.dq_row_sumsq.restype = st
    lib.dq_quantize_pack_asym.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp]
    lib.dq_quantize_pack_asym.restype = st
    lib.dq_unpack_asym.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp]
    lib.dq_unpack_asym.restype = st
    lib.dq_gemv_asym.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, vp, vp]
    lib.dq_gemv_asym.restype = st
    lib.dq_gemm_asym.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, vp, vp]
    lib.dq_gemm_asym.restype = st
    lib.dq_quantize_pack_group.argtypes = [vp, i32, i64, i64, i32, i64, vp, vp, vp]
    lib.dq_quantize_pack_group.restype = st
    lib.dq_unpack_group.argtypes = [vp, vp, i64, i64, i32, i64, vp, vp, vp]
    lib.dq_unpack_group.restype = st
    lib.dq_gemv_group.argtypes = [vp, i64, vp, vp, i64, i64, i32, i64, vp, vp]
    lib.dq_gemv_group.restype = st
    lib.dq_gemm_group.argtypes = [vp, i64, vp, vp, i64, i64, i32, i64, vp, vp]
    lib.dq_gemm_group.restype = st
    fp = ctypes.POINTER(DQFileMatrix)
    lib.dq_file_write.argtypes = [ctypes.c_char_p, fp, i64]
    lib.dq_file_write.restype = st
    lib.dq_file_open.argtypes = [ctypes.c_char_p, ctypes.POINTER(vp)]
    lib.dq_file_open.restype = st
    lib.dq_file_count.argtypes = [vp]
    lib.dq_file_count.restype = i64
    lib.dq_file_matrix_info.argtypes = [vp, i64, fp]
    lib.dq_file_matrix_info.restype = st
    lib.dq_file_verify.argtypes = [vp, i64]
    lib.dq_file_verify.restype = st
    lib.dq_file_load.argtypes = [vp, i64, vp, vp, vp]
    lib.dq_file_load.restype = st
    lib.dq_file_close.argtypes = [vp]
    lib.dq_file_close.restype = None
    lib.dq_quantize_pack_sumsq.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.dq_quantize_pack_sumsq.restype = st
    lib.dq_sensitivity.argtypes = [vp, vp, vp, i64, vp]
    lib.dq_sensitivity.restype = st
    lib.dq_allocate_bits.argtypes = [vp, vp, i64, vp, i32, i64, vp, vp, vp, i64, vp, vp]
    lib.dq_allocate_bits.restype = st
    lib.dq_status_string.argtypes = [st]
    lib.dq_status_string.restype = ctypes.c_char_p
    lib.dq_last_error.argtypes = []
    lib.dq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------- raw C ABI

def dq_packed_row_bytes(K: int, bits: int) -> int:
    return int(load().dq_packed_row_bytes(K, bits))


def dq_quantize_pack(w: int, w_dtype: int, N: int, K: int, bits: int, packed: int, scales: int,
                     nonfinite_rows: int = 0, stream: int = 0) -> int:
    return int(load().dq_quantize_pack(w, w_dtype, N, K, bits, packed, scales, nonfinite_rows,
                                       stream))


def dq_quantize_pack_asym(w: int, w_dtype: int, N: int, K: int, bits: int, packed: int,
                          scales: int, zeros: int, stream: int = 0) -> int:
    return int(load().dq_quantize_pack_asym(w, w_dtype, N, K, bits, packed, scales, zeros, stream))


def dq_unpack_asym(packed: int, scales: int, zeros: int, N: int, K: int, bits: int, q_out: int,
                   w_out: int, stream: int = 0) -> int:
    return int(load().dq_unpack_asym(packed, scales, zeros, N, K, bits, q_out, w_out, stream))


def dq_gemv_asym(x: int, M: int, packed: int, scales: int, zeros: int, N: int, K: int,
                 bits: int, y: int, stream: int = 0) -> int:
    return int(load().dq_gemv_asym(x, M, packed, scales, zeros, N, K, bits, y, stream))


def dq_gemm_asym(x: int, M: int, packed: int, scales: int, zeros: int, N: int, K: int,
                 bits: int, y: int, stream: int = 0) -> int:
    return int(load().dq_gemm_asym(x, M, packed, scales, zeros, N, K, bits, y, stream))


def dq_quantize_pack_group(w: int, w_dtype: int, N: int, K: int, bits: int, group: int,
                           packed: int, scales: int, stream: int = 0) -> int:
    return int(load().dq_quantize_pack_group(w, w_dtype, N, K, bits, group, packed, scales, stream))


def dq_unpack_group(packed: int, scales: int, N: int, K: int, bits: int, group: int, q_out: int,
                    w_out: int, stream: int = 0) -> int:
    return int(load().dq_unpack_group(packed, scales, N, K, bits, group, q_out, w_out, stream))


def dq_gemv_group(x: int, M: int, packed: int, scales: int, N: int, K: int, bits: int, group: int,
                  y: int, stream: int = 0) -> int:
    return int(load().dq_gemv_group(x, M, packed, scales, N, K, bits, group, y, stream))


def dq_gemm_group(x: int, M: int, packed: int, scales: int, N: int, K: int, bits: int, group: int,
                  y: int, stream: int = 0) -> int:
    return int(load().dq_gemm_group(x, M, packed, scales, N, K, bits, group, y, stream))


def dq_row_sumsq(w: int, w_dtype: int, N: int, K: int, row_sumsq: int, matrix_sumsq: int,
                 stream: int = 0) -> int:
    return int(load().dq_row_sumsq(w, w_dtype, N, K, row_sumsq, matrix_sumsq, stream))


def dq_quantize_pack_sumsq(w: int, w_dtype: int, N: int, K: int, bits: int, packed: int,
                           scales: int, row_sumsq: int, matrix_sumsq: int, stream: int = 0) -> int:
    return int(load().dq_quantize_pack_sumsq(w, w_dtype, N, K, bits, packed, scales, row_sumsq,
                                             matrix_sumsq, stream))


def dq_sensitivity(h_trace: int, sumsq: int, params: int, n: int, out: int) -> int:
    return int(load().dq_sensitivity(h_trace, sumsq, params, n, out))


def dq_allocate_bits(sensitivity: int, params: int, n: int, levels: int, n_levels: int,
                     budget_bits: int, bits_out: int, step_matrix: int, step_bits: int,
                     step_capacity: int, n_steps: int, loss: int) -> int:
    return int(load().dq_allocate_bits(sensitivity, params, n, levels, n_levels, budget_bits,
                                       bits_out, step_matrix, step_bits, step_capacity, n_steps,
                                       loss))


def dq_unpack(packed: int, scales: int, N: int, K: int, bits: int, q_out: int, w_out: int,
              stream: int = 0) -> int:
    return int(load().dq_unpack(packed, scales, N, K, bits, q_out, w_out, stream))


def dq_gemv(x: int, M: int, packed: int, scales: int, N: int, K: int, bits: int, y: int,
            stream: int = 0) -> int:
    return int(load().dq_gemv(x, M, packed, scales, N, K, bits, y, stream))


def dq_gemv_batched(items: int, count: int, M: int, stream: int = 0) -> int:
    """items: address of a host array of ``DQGemvItem``."""
    return int(load().dq_gemv_batched(items, count, M, stream))


def dq_gemm(x: int, M: int, packed: int, scales: int, N: int, K: int, bits: int, y: int,
            stream: int = 0) -> int:
    return int(load().dq_gemm(x, M, packed, scales, N, K, bits, y, stream))


def dq_stream_read(buf: int, nbytes: int, partial: int, nparts: int, stream: int = 0) -> int:
    return int(load().dq_stream_read(buf, nbytes, partial, nparts, stream))


def dq_status_string(status: int) -> str:
    return load().dq_status_string(status).decode()


def dq_last_error() -> str:
    return load().dq_last_error().decode()


# ----------------------------------------------------------- torch tensors

def packed_row_bytes(K: int, bits: int) -> int:
    rb = dq_packed_row_bytes(K, bits)
    if rb == 0:
        raise DQError(DQ_ERR_SHAPE if 2 <= bits <= 15 else DQ_ERR_BITS, "packed_row_bytes")
    return rb


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtypes, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s dtype %s not in %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-D tensor" % (name, ndim))


def _check(status: int, where: str):
    if status != DQ_OK:
        raise DQError(status, where)


def quantize_pack(w, bits: int, packed=None, scales=None, nonfinite=None):
    """W[N, K] (float32 or bfloat16, on the GPU) -> (packed int32 [N, row_bytes/4] holding
    the uint32 words, scales float32 [N]).  nonfinite: optional int32 [1] tensor
    that receives the number of rows holding a NaN or an infinity."""
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16), 2)
    N, K = w.shape
    rw = packed_row_bytes(K, bits) // 4
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((N,), dtype=torch.float32, device=w.device)
    _need(packed, "packed", (torch.int32,), 2)
    _need(scales, "scales", (torch.float32,), 1)
    if tuple(packed.shape) != (N, rw) or tuple(scales.shape) != (N,):
        raise ValueError("packed/scales shape mismatch")
    if nonfinite is not None:
        _need(nonfinite, "nonfinite", (torch.int32,), 1)
        if nonfinite.shape[0] != 1:
            raise ValueError("nonfinite must be [1]")
    dt = DQ_BF16 if w.dtype == torch.bfloat16 else DQ_F32
    _check(dq_quantize_pack(w.data_ptr(), dt, N, K, bits, packed.data_ptr(), scales.data_ptr(),
                            nonfinite.data_ptr() if nonfinite is not None else 0, _stream(w)),
           "dq_quantize_pack")
    return packed, scales


def quantize_pack_asym(w, bits: int):
    """Asymmetric per-row quantization: W[N, K] (float32 / bfloat16, GPU) ->
    (packed int32 [N, row_words] holding unsigned codes, scales float32 [N],
    zeros int32 [N])."""
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16), 2)
    N, K = w.shape
    packed = torch.empty((N, packed_row_bytes(K, bits) // 4), dtype=torch.int32, device=w.device)
    scales = torch.empty((N,), dtype=torch.float32, device=w.device)
    zeros = torch.empty((N,), dtype=torch.int32, device=w.device)
    dt = DQ_BF16 if w.dtype == torch.bfloat16 else DQ_F32
    _check(dq_quantize_pack_asym(w.data_ptr(), dt, N, K, bits, packed.data_ptr(), scales.data_ptr(),
                                 zeros.data_ptr(), _stream(w)), "dq_quantize_pack_asym")
    return packed, scales, zeros


def unpack_asym(packed, scales, zeros, K: int, bits: int, want_q: bool = True,
                want_w: bool = False):
    """(q = u - z int32 [N, K] or None, w_hat float32 [N, K] or None)."""
    torch = _torch()
    _need(packed, "packed", (torch.int32,), 2)
    _need(zeros, "zeros", (torch.int32,), 1)
    N = packed.shape[0]
    if packed.shape[1] != packed_row_bytes(K, bits) // 4 or zeros.shape[0] != N:
        raise ValueError("packed / zeros do not match N, K and bits")
    q = torch.empty((N, K), dtype=torch.int32, device=packed.device) if want_q else None
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device) if want_w else None
    if scales is not None:
        _need(scales, "scales", (torch.float32,), 1)
    _check(dq_unpack_asym(packed.data_ptr(), scales.data_ptr() if scales is not None else 0,
                          zeros.data_ptr(), N, K, bits, q.data_ptr() if q is not None else 0,
                          w.data_ptr() if w is not None else 0, _stream(packed)), "dq_unpack_asym")
    return q, w


def _matmul_asym(fn, name, x, packed, scales, zeros, K: int, bits: int, y=None):
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(packed, "packed", (torch.int32,), 2)
    _need(scales, "scales", (torch.float32,), 1)
    _need(zeros, "zeros", (torch.int32,), 1)
    M, N = x.shape[0], packed.shape[0]
    if (x.shape[1] != K or packed.shape[1] != packed_row_bytes(K, bits) // 4
            or scales.shape[0] != N or zeros.shape[0] != N):
        raise ValueError("shape mismatch between x, packed, scales, zeros, K and bits")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    _check(fn(x.data_ptr(), M, packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, bits,
              y.data_ptr(), _stream(x)), name)
    return y


def gemv_asym(x, packed, scales, zeros, K: int, bits: int, y=None):
    """y = s * x . (u - z)^T for 1 <= M <= 16."""
    return _matmul_asym(dq_gemv_asym, "dq_gemv_asym", x, packed, scales, zeros, K, bits, y)


def gemm_asym(x, packed, scales, zeros, K: int, bits: int, y=None):
    """y = s * x . (u - z)^T on the matrix cores (any M >= 1)."""
    return _matmul_asym(dq_gemm_asym, "dq_gemm_asym", x, packed, scales, zeros, K, bits, y)


def quantize_pack_group(w, bits: int, group: int):
    """Group-wise scales: W[N, K] -> (packed int32 [N, row_words], scales float32
    [N, ceil(K / group)])."""
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16), 2)
    N, K = w.shape
    packed = torch.empty((N, packed_row_bytes(K, bits) // 4), dtype=torch.int32, device=w.device)
    scales = torch.empty((N, -(-K // group)), dtype=torch.float32, device=w.device)
    dt = DQ_BF16 if w.dtype == torch.bfloat16 else DQ_F32
    _check(dq_quantize_pack_group(w.data_ptr(), dt, N, K, bits, group, packed.data_ptr(),
                                  scales.data_ptr(), _stream(w)), "dq_quantize_pack_group")
    return packed, scales


def unpack_group(packed, scales, K: int, bits: int, group: int, want_q: bool = True,
                 want_w: bool = False):
    torch = _torch()
    _need(packed, "packed", (torch.int32,), 2)
    N = packed.shape[0]
    if packed.shape[1] != packed_row_bytes(K, bits) // 4:
        raise ValueError("packed row length does not match K and bits")
    if scales is not None:
        _need(scales, "scales", (torch.float32,), 2)
        if tuple(scales.shape) != (N, -(-K // group)):
            raise ValueError("scales must be [N, ceil(K / group)]")
    q = torch.empty((N, K), dtype=torch.int32, device=packed.device) if want_q else None
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device) if want_w else None
    _check(dq_unpack_group(packed.data_ptr(), scales.data_ptr() if scales is not None else 0, N, K,
                           bits, group, q.data_ptr() if q is not None else 0,
                           w.data_ptr() if w is not None else 0, _stream(packed)),
           "dq_unpack_group")
    return q, w


def _matmul_group(fn, name, x, packed, scales, K: int, bits: int, group: int, y=None):
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(packed, "packed", (torch.int32,), 2)
    _need(scales, "scales", (torch.float32,), 2)
    M, N = x.shape[0], packed.shape[0]
    if (x.shape[1] != K or packed.shape[1] != packed_row_bytes(K, bits) // 4
            or tuple(scales.shape) != (N, -(-K // group))):
        raise ValueError("shape mismatch between x, packed, scales, K, bits and group")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    _check(fn(x.data_ptr(), M, packed.data_ptr(), scales.data_ptr(), N, K, bits, group,
              y.data_ptr(), _stream(x)), name)
    return y


def gemv_group(x, packed, scales, K: int, bits: int, group: int, y=None):
    """y = sum_k x q s[n, k / group] for 1 <= M <= 16."""
    return _matmul_group(dq_gemv_group, "dq_gemv_group", x, packed, scales, K, bits, group, y)


def gemm_group(x, packed, scales, K: int, bits: int, group: int, y=None):
    """The same on the bf16 matrix cores (any M >= 1)."""
    return _matmul_group(dq_gemm_group, "dq_gemm_group", x, packed, scales, K, bits, group, y)


def row_sumsq(w, want_total: bool = True):
    """fp64 sum of w^2 of every row of W[N, K] (float32 or bfloat16, on the GPU),
    and of the whole matrix.  Returns (row_sumsq float64 [N], matrix_sumsq float64
    [1] or None)."""
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16), 2)
    N, K = w.shape
    row = torch.empty((N,), dtype=torch.float64, device=w.device)
    total = torch.empty((1,), dtype=torch.float64, device=w.device) if want_total else None
    dt = DQ_BF16 if w.dtype == torch.bfloat16 else DQ_F32
    _check(dq_row_sumsq(w.data_ptr(), dt, N, K, row.data_ptr(),
                        total.data_ptr() if total is not None else 0, _stream(w)), "dq_row_sumsq")
    return row, total


def quantize_pack_sumsq(w, bits: int, want_total: bool = True):
    """``quantize_pack`` plus the fp64 sum of w^2 of every row, taken in the same
    pass.  Returns (packed, scales, row_sumsq float64 [N], matrix_sumsq float64 [1]
    or None)."""
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16), 2)
    N, K = w.shape
    rw = packed_row_bytes(K, bits) // 4
    packed = torch.empty((N, rw), dtype=torch.int32, device=w.device)
    scales = torch.empty((N,), dtype=torch.float32, device=w.device)
    row = torch.empty((N,), dtype=torch.float64, device=w.device)
    total = torch.empty((1,), dtype=torch.float64, device=w.device) if want_total else None
    dt = DQ_BF16 if w.dtype == torch.bfloat16 else DQ_F32
    _check(dq_quantize_pack_sumsq(w.data_ptr(), dt, N, K, bits, packed.data_ptr(),
                                  scales.data_ptr(), row.data_ptr(),
                                  total.data_ptr() if total is not None else 0, _stream(w)),
           "dq_quantize_pack_sumsq")
    return packed, scales, row, total


def _host(a, dtype, name):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=dtype)
    if a.ndim != 1:
        raise ValueError("%s must be 1-D" % name)
    return a


def _addr(a) -> int:
    return a.ctypes.data


def sensitivity(h_trace, sumsq, params):
    """Sensitivity per matrix, h_trace * (sumsq / params), on the host (numpy in,
    numpy float64 out)."""
    import numpy as np
    h = _host(h_trace, np.float64, "h_trace")
    ss = _host(sumsq, np.float64, "sumsq")
    p = _host(params, np.int64, "params")
    if not h.size == ss.size == p.size:
        raise ValueError("h_trace, sumsq and params must have one entry per matrix")
    out = np.empty(h.size, dtype=np.float64)
    _check(dq_sensitivity(_addr(h), _addr(ss), _addr(p), h.size, _addr(out)), "dq_sensitivity")
    return out


def allocate_bits(sens, params, levels=FULL_LEVELS, budget_bits=None):
    """Water-filling allocation on the host.  Returns (bits int32 [n], steps as a
    list of (matrix, new width) in the order taken, predicted loss).  A budget
    of None walks the whole frontier."""
    import numpy as np
    s = _host(sens, np.float64, "sensitivity")
    p = _host(params, np.int64, "params")
    lv = _host(levels, np.int32, "levels")
    if s.size != p.size:
        raise ValueError("one sensitivity and one parameter count per matrix")
    bits = np.empty(s.size, dtype=np.int32)
    cap = s.size * max(lv.size - 1, 0)
    sm = np.empty(max(cap, 1), dtype=np.int64)
    sb = np.empty(max(cap, 1), dtype=np.int32)
    nsteps = np.zeros(1, dtype=np.int64)
    loss = np.zeros(1, dtype=np.float64)
    budget = -1 if budget_bits is None else int(budget_bits)
    if budget_bits is not None and budget < 0:
        raise ValueError("budget_bits must be >= 0 (None = no limit)")
    _check(dq_allocate_bits(_addr(s), _addr(p), s.size, _addr(lv), lv.size, budget, _addr(bits),
                            _addr(sm), _addr(sb), cap, _addr(nsteps), _addr(loss)),
           "dq_allocate_bits")
    n = int(nsteps[0])
    return bits, list(zip(sm[:n].tolist(), sb[:n].tolist())), float(loss[0])


def unpack(packed, scales, K: int, bits: int, want_q: bool = True, want_w: bool = False):
    """packed [N, row_words] -> (q int32 [N, K] or None, w_hat float32 [N, K] or None)."""
    torch = _torch()
    _need(packed, "packed", (torch.int32,), 2)
    N = packed.shape[0]
    if packed.shape[1] != packed_row_bytes(K, bits) // 4:
        raise ValueError("packed row length does not match K and bits")
    q = torch.empty((N, K), dtype=torch.int32, device=packed.device) if want_q else None
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device) if want_w else None
    if scales is not None:
        _need(scales, "scales", (torch.float32,), 1)
    _check(dq_unpack(packed.data_ptr(), scales.data_ptr() if scales is not None else 0, N, K, bits,
                     q.data_ptr() if q is not None else 0, w.data_ptr() if w is not None else 0,
                     _stream(packed)), "dq_unpack")
    return q, w


def _matmul(fn, name, x, packed, scales, K: int, bits: int, y=None):
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(packed, "packed", (torch.int32,), 2)
    _need(scales, "scales", (torch.float32,), 1)
    M = x.shape[0]
    N = packed.shape[0]
    if x.shape[1] != K or packed.shape[1] != packed_row_bytes(K, bits) // 4 or scales.shape[0] != N:
        raise ValueError("shape mismatch between x, packed, scales, K and bits")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    _check(fn(x.data_ptr(), M, packed.data_ptr(), scales.data_ptr(), N, K, bits, y.data_ptr(),
              _stream(x)), name)
    return y


def gemv(x, packed, scales, K: int, bits: int, y=None):
    """y[M, N] = x . dequant(W)^T for 1 <= M <= 16 (fp32 accumulate)."""
    return _matmul(dq_gemv, "dq_gemv", x, packed, scales, K, bits, y)


def gemv_batched(items, ys=None):
    """Several decode products in one call: items is a list of (x, packed,
    scales, K, bits), optionally followed by zeros (int32 [N] zero points of
    asymmetric codes, or None) and group (codes per group scale, scales then
    [N, ceil(K / group)]; 0 for a scale per row); bf16 x [M, K] with the same
    M for all; x and weights may be shared between items.  Returns the list of
    y [M, N] (or fills ``ys``).  The items of each scheme that fit one launch
    share it; the others run as one launch each of their scheme's entry point."""
    torch = _torch()
    if not 1 <= len(items) <= GEMV_BATCH_MAX:
        raise ValueError("1 to %d items" % GEMV_BATCH_MAX)
    arr = (DQGemvItem * len(items))()
    out = []
    M = None
    for i, item in enumerate(items):
        if not 5 <= len(item) <= 7:
            raise ValueError("item %d: (x, packed, scales, K, bits[, zeros[, group]])" % i)
        x, packed, scales, K, bits = item[:5]
        zeros = item[5] if len(item) > 5 else None
        group = item[6] if len(item) > 6 else 0
        _need(x, "x", (torch.bfloat16,), 2)
        _need(packed, "packed", (torch.int32,), 2)
        N = packed.shape[0]
        if group:
            _need(scales, "scales", (torch.float32,), 2)
            ok_scales = tuple(scales.shape) == (N, -(-K // group))
        else:
            _need(scales, "scales", (torch.float32,), 1)
            ok_scales = scales.shape[0] == N
        if zeros is not None:
            _need(zeros, "zeros", (torch.int32,), 1)
            ok_scales = ok_scales and zeros.shape[0] == N
        if M is None:
            M = x.shape[0]
        if x.shape[0] != M or x.shape[1] != K or \
                packed.shape[1] != packed_row_bytes(K, bits) // 4 or not ok_scales:
            raise ValueError("item %d: shape mismatch between x, packed, scales, zeros, K and bits" % i)
        y = ys[i] if ys is not None else torch.empty((M, N), dtype=torch.float32, device=x.device)
        _need(y, "y", (torch.float32,), 2)
        if tuple(y.shape) != (M, N):
            raise ValueError("item %d: y must be [M, N]" % i)
        arr[i] = DQGemvItem(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), y.data_ptr(), N, K,
                            bits, group, zeros.data_ptr() if zeros is not None else 0)
        out.append(y)
    _check(dq_gemv_batched(ctypes.addressof(arr), len(items), M, _stream(items[0][0])),
           "dq_gemv_batched")
    return out


def gemm(x, packed, scales, K: int, bits: int, y=None):
    """y[M, N] = x . dequant(W)^T on the bf16 matrix cores (any M >= 1)."""
    return _matmul(dq_gemm, "dq_gemm", x, packed, scales, K, bits, y)


def stream_read(buf, nparts: int, partial=None):
    """Plain streaming read of a contiguous GPU tensor (any dtype, a multiple of
    16 bytes): the yardstick for the bandwidth-bound calls, not a step of the
    method.  Returns int32 [nparts] whose XOR is the XOR of every 32-bit word."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if partial is None:
        partial = torch.empty((nparts,), dtype=torch.int32, device=buf.device)
    _need(partial, "partial", (torch.int32,), 1)
    if partial.shape[0] != nparts:
        raise ValueError("partial must hold nparts words")
    nbytes = buf.numel() * buf.element_size()
    _check(dq_stream_read(buf.data_ptr(), nbytes, partial.data_ptr(), nparts, _stream(buf)),
           "dq_stream_read")
    return partial


# ------------------------------------------------------ on-disk packed format

def write_packed_file(path: str, matrices) -> None:
    """Write matrices to a packed-weight file.  ``matrices``: (name, N, K, bits,
    data, scales) with host numpy arrays -- data the packed words [N, row_words]
    (any 4-byte dtype) for bits 2..15, or bf16 bit patterns [N, K] (uint16) for
    bits 16; scales float32 [N] (None for bits 16)."""
    import numpy as np
    keep = []
    arr = (DQFileMatrix * len(matrices))()
    for i, (name, N, K, bits, data, scales) in enumerate(matrices):
        raw = name.encode("utf-8")
        if len(raw) > 63 or b"\0" in raw:
            raise ValueError("a name takes at most 63 UTF-8 bytes and no NUL")
        data = np.ascontiguousarray(data)
        want = N * (K * 2 if bits == 16 else dq_packed_row_bytes(K, bits))
        if data.nbytes != want:
            raise ValueError("matrix %r: data holds %d bytes, %d expected" % (name, data.nbytes, want))
        arr[i].name = raw
        arr[i].N, arr[i].K, arr[i].bits = N, K, bits
        arr[i].data = data.ctypes.data
        if scales is not None:
            scales = np.ascontiguousarray(scales, dtype=np.float32)
            if scales.shape != (N,):
                raise ValueError("matrix %r: scales must be float32 [N]" % name)
            arr[i].scales = scales.ctypes.data
        keep.append((data, scales))
    _check(int(load().dq_file_write(path.encode(), arr, len(matrices))), "dq_file_write")


class PackedFile:
    """A packed-weight file mapped read-only (``dq_file_open``); use as a
    context manager or call ``close``."""

    def __init__(self, path: str):
        h = ctypes.c_void_p()
        _check(int(load().dq_file_open(path.encode(), ctypes.byref(h))), "dq_file_open")
        self._h = h

    def __len__(self):
        return int(load().dq_file_count(self._h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def close(self):
        if self._h:
            load().dq_file_close(self._h)
            self._h = ctypes.c_void_p()

    def info(self, i: int):
        """(name, N, K, bits, data, scales): numpy views into the mapping (valid
        until ``close``); data is uint32 [N, row_words] or uint16 (bf16) [N, K]."""
        import numpy as np
        m = DQFileMatrix()
        _check(int(load().dq_file_matrix_info(self._h, i, ctypes.byref(m))), "dq_file_matrix_info")
        N, K, bits = int(m.N), int(m.K), int(m.bits)
        if bits == 16:
            data = np.ctypeslib.as_array(ctypes.cast(m.data, ctypes.POINTER(ctypes.c_uint16)),
                                         shape=(N, K))
            scales = None
        else:
            rw = dq_packed_row_bytes(K, bits) // 4
            data = np.ctypeslib.as_array(ctypes.cast(m.data, ctypes.POINTER(ctypes.c_uint32)),
                                         shape=(N, rw))
            scales = np.ctypeslib.as_array(ctypes.cast(m.scales, ctypes.POINTER(ctypes.c_float)),
                                           shape=(N,))
        return m.name.decode("utf-8"), N, K, bits, data, scales

    def verify(self, i: int) -> bool:
        st = int(load().dq_file_verify(self._h, i))
        if st == DQ_ERR_FORMAT:
            return False
        _check(st, "dq_file_verify")
        return True

    def load(self, i: int, device="cuda"):
        """Copy entry i into new GPU tensors: (packed int32 [N, row_words], scales
        float32 [N]) for bits 2..15, (bf16 [N, K], None) for bits 16.  Waits for
        the copy, so the tensors are ready when it returns."""
        torch = _torch()
        name, N, K, bits, _, _ = self.info(i)
        dev = torch.device(device)
        if bits == 16:
            data = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            scales = None
        else:
            data = torch.empty((N, dq_packed_row_bytes(K, bits) // 4), dtype=torch.int32, device=dev)
            scales = torch.empty((N,), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev)
        _check(int(load().dq_file_load(self._h, i, data.data_ptr(),
                                       scales.data_ptr() if scales is not None else 0,
                                       stream.cuda_stream)), "dq_file_load")
        stream.synchronize()
        return data, scales
