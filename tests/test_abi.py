"""The C ABI without a GPU: the library loads, exports every entry point that
include/dq.h declares, sizes rows as documented, and rejects every invalid
argument on the host before any HIP call (so these run on a CPU-only machine:
the fake device addresses below are never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import mixed_precision_weight_dq_amd as dq
from pins import row_bytes_formula

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dq.h")

A = 1 << 20  # a 16-byte aligned fake device address; never touched
MIS = A + 4  # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dq_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("dq_packed_row_bytes", "dq_quantize_pack", "dq_unpack", "dq_gemv", "dq_gemm",
                 "dq_status_string", "dq_last_error", "dq_quantize_pack_sumsq", "dq_sensitivity",
                 "dq_row_sumsq", "dq_quantize_pack_asym", "dq_unpack_asym",
                 "dq_gemv_asym", "dq_gemm_asym", "dq_quantize_pack_group", "dq_unpack_group",
                 "dq_gemv_group", "dq_gemm_group", "dq_file_write", "dq_file_open", "dq_file_count",
                 "dq_file_matrix_info", "dq_file_verify", "dq_file_load", "dq_file_close",
                 "dq_allocate_bits"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dq.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_row_bytes():
    for bits in range(2, 16):
        for K in (1, 2, 31, 32, 33, 255, 256, 614, 4096, 5120, 8192, 17408, 1 << 22):
            assert dq.dq_packed_row_bytes(K, bits) == row_bytes_formula(K, bits)
    assert dq.dq_packed_row_bytes(0, 4) == 0
    assert dq.dq_packed_row_bytes((1 << 22) + 1, 4) == 0
    assert dq.dq_packed_row_bytes(64, 1) == 0
    assert dq.dq_packed_row_bytes(64, 16) == 0


def test_status_strings():
    for s in range(11):
        assert dq.dq_status_string(s) != "unknown status"
    assert dq.dq_status_string(99) == "unknown status"
    assert dq.dq_last_error() == ""


@pytest.mark.parametrize("bits", [0, 1, 16, 32, -3])
def test_bits_rejected(bits):
    assert dq.dq_quantize_pack(A, dq.DQ_BF16, 4, 64, bits, A, A) == dq.DQ_ERR_BITS
    assert dq.dq_unpack(A, A, 4, 64, bits, A, 0) == dq.DQ_ERR_BITS
    assert dq.dq_gemv(A, 1, A, A, 4, 64, bits, A) == dq.DQ_ERR_BITS
    assert dq.dq_gemm(A, 1, A, A, 4, 64, bits, A) == dq.DQ_ERR_BITS


@pytest.mark.parametrize("N,K", [(0, 64), (4, 0), (-1, 64), (4, -5), (1 << 31, 64),
                                 (4, (1 << 22) + 1)])
def test_shape_rejected(N, K):
    assert dq.dq_quantize_pack(A, dq.DQ_F32, N, K, 6, A, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_unpack(A, A, N, K, 6, A, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_gemv(A, 1, A, A, N, K, 6, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_gemm(A, 1, A, A, N, K, 6, A) == dq.DQ_ERR_SHAPE


@pytest.mark.parametrize("M", [0, -1, 17, 1000])
def test_gemv_m_rejected(M):
    assert dq.dq_gemv(A, M, A, A, 4, 64, 6, A) == dq.DQ_ERR_SHAPE


@pytest.mark.parametrize("M", [0, -2, 1 << 31])
def test_gemm_m_rejected(M):
    assert dq.dq_gemm(A, M, A, A, 4, 64, 6, A) == dq.DQ_ERR_SHAPE


def test_null_rejected():
    assert dq.dq_quantize_pack(0, dq.DQ_BF16, 4, 64, 6, A, A) == dq.DQ_ERR_NULL
    assert dq.dq_quantize_pack(A, dq.DQ_BF16, 4, 64, 6, 0, A) == dq.DQ_ERR_NULL
    assert dq.dq_quantize_pack(A, dq.DQ_BF16, 4, 64, 6, A, 0) == dq.DQ_ERR_NULL
    assert dq.dq_unpack(0, A, 4, 64, 6, A, A) == dq.DQ_ERR_NULL
    assert dq.dq_unpack(A, A, 4, 64, 6, 0, 0) == dq.DQ_ERR_NULL  # no output requested
    assert dq.dq_unpack(A, 0, 4, 64, 6, 0, A) == dq.DQ_ERR_NULL  # w_out needs scales
    for fn in (dq.dq_gemv, dq.dq_gemm):
        assert fn(0, 1, A, A, 4, 64, 6, A) == dq.DQ_ERR_NULL
        assert fn(A, 1, 0, A, 4, 64, 6, A) == dq.DQ_ERR_NULL
        assert fn(A, 1, A, 0, 4, 64, 6, A) == dq.DQ_ERR_NULL
        assert fn(A, 1, A, A, 4, 64, 6, 0) == dq.DQ_ERR_NULL


def test_dtype_rejected():
    for dt in (-1, 2, 7):
        assert dq.dq_quantize_pack(A, dt, 4, 64, 6, A, A) == dq.DQ_ERR_DTYPE


def test_alignment_rejected():
    assert dq.dq_quantize_pack(MIS, dq.DQ_F32, 4, 64, 6, A, A) == dq.DQ_ERR_ALIGN
    assert dq.dq_quantize_pack(A, dq.DQ_F32, 4, 64, 6, MIS, A) == dq.DQ_ERR_ALIGN
    assert dq.dq_quantize_pack(A, dq.DQ_F32, 4, 64, 6, A, A + 2) == dq.DQ_ERR_ALIGN
    assert dq.dq_quantize_pack(A, dq.DQ_F32, 4, 64, 6, A, A, A + 2) == dq.DQ_ERR_ALIGN
    assert dq.dq_unpack(MIS, A, 4, 64, 6, A, 0) == dq.DQ_ERR_ALIGN
    assert dq.dq_unpack(A, A, 4, 64, 6, A + 1, 0) == dq.DQ_ERR_ALIGN
    for fn in (dq.dq_gemv, dq.dq_gemm):
        assert fn(MIS, 1, A, A, 4, 64, 6, A) == dq.DQ_ERR_ALIGN
        assert fn(A, 1, MIS, A, 4, 64, 6, A) == dq.DQ_ERR_ALIGN
        assert fn(A, 1, A, A + 2, 4, 64, 6, A) == dq.DQ_ERR_ALIGN
        assert fn(A, 1, A, A, 4, 64, 6, A + 2) == dq.DQ_ERR_ALIGN


def test_stream_read_arguments_rejected():
    assert dq.dq_stream_read(0, 64, A, 1) == dq.DQ_ERR_NULL
    assert dq.dq_stream_read(A, 64, 0, 1) == dq.DQ_ERR_NULL
    for nbytes in (0, 8, 24, -16):
        assert dq.dq_stream_read(A, nbytes, A, 1) == dq.DQ_ERR_SHAPE
    for nparts in (0, -1, 65537):
        assert dq.dq_stream_read(A, 64, A, nparts) == dq.DQ_ERR_SHAPE
    assert dq.dq_stream_read(A + 8, 64, A, 1) == dq.DQ_ERR_ALIGN
    assert dq.dq_stream_read(A, 64, A + 2, 1) == dq.DQ_ERR_ALIGN


def test_tensor_wrappers_refuse_cpu_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        dq.quantize_pack(w, 6)
    with pytest.raises(dq.DQError):
        dq.packed_row_bytes(64, 1)


def test_quantize_pack_sumsq_arguments_rejected():
    f = dq.dq_quantize_pack_sumsq
    assert f(A, dq.DQ_BF16, 4, 64, 6, A, A, 0, A) == dq.DQ_ERR_NULL   # row sums required
    assert f(0, dq.DQ_BF16, 4, 64, 6, A, A, A, 0) == dq.DQ_ERR_NULL
    assert f(A, dq.DQ_BF16, 4, 64, 16, A, A, A, 0) == dq.DQ_ERR_BITS
    assert f(A, dq.DQ_BF16, 0, 64, 6, A, A, A, 0) == dq.DQ_ERR_SHAPE
    assert f(A, 3, 4, 64, 6, A, A, A, 0) == dq.DQ_ERR_DTYPE
    assert f(A, dq.DQ_BF16, 4, 64, 6, A, A, A + 4, 0) == dq.DQ_ERR_ALIGN
    assert f(A, dq.DQ_BF16, 4, 64, 6, A, A, A, A + 4) == dq.DQ_ERR_ALIGN
    assert f(MIS, dq.DQ_BF16, 4, 64, 6, A, A, A, 0) == dq.DQ_ERR_ALIGN


def test_row_sumsq_arguments_rejected():
    f = dq.dq_row_sumsq
    assert f(0, dq.DQ_BF16, 4, 64, A, 0) == dq.DQ_ERR_NULL
    assert f(A, dq.DQ_BF16, 4, 64, 0, A) == dq.DQ_ERR_NULL
    for N, K in ((0, 64), (4, 0), (1 << 31, 64), (4, (1 << 22) + 1)):
        assert f(A, dq.DQ_F32, N, K, A, 0) == dq.DQ_ERR_SHAPE
    assert f(A, 2, 4, 64, A, 0) == dq.DQ_ERR_DTYPE
    assert f(MIS, dq.DQ_F32, 4, 64, A, 0) == dq.DQ_ERR_ALIGN
    assert f(A, dq.DQ_F32, 4, 64, A + 4, 0) == dq.DQ_ERR_ALIGN
    assert f(A, dq.DQ_F32, 4, 64, A, A + 4) == dq.DQ_ERR_ALIGN


def test_asym_arguments_rejected():
    q = dq.dq_quantize_pack_asym
    assert q(A, dq.DQ_BF16, 4, 64, 6, A, A, 0) == dq.DQ_ERR_NULL
    assert q(A, dq.DQ_BF16, 4, 64, 16, A, A, A) == dq.DQ_ERR_BITS
    assert q(A, dq.DQ_BF16, 0, 64, 6, A, A, A) == dq.DQ_ERR_SHAPE
    assert q(A, 9, 4, 64, 6, A, A, A) == dq.DQ_ERR_DTYPE
    assert q(A, dq.DQ_BF16, 4, 64, 6, A, A, A + 2) == dq.DQ_ERR_ALIGN
    u = dq.dq_unpack_asym
    assert u(A, A, 0, 4, 64, 6, A, 0) == dq.DQ_ERR_NULL
    assert u(A, 0, A, 4, 64, 6, 0, A) == dq.DQ_ERR_NULL  # w_out needs scales
    assert u(A, A, A + 1, 4, 64, 6, A, 0) == dq.DQ_ERR_ALIGN
    for fn, bad_m in ((dq.dq_gemv_asym, 17), (dq.dq_gemm_asym, 0)):
        assert fn(A, 1, A, A, 0, 4, 64, 6, A) == dq.DQ_ERR_NULL
        assert fn(A, 1, A, A, A, 4, 64, 6, 0) == dq.DQ_ERR_NULL
        assert fn(A, bad_m, A, A, A, 4, 64, 6, A) == dq.DQ_ERR_SHAPE
        assert fn(A, 1, A, A, A, 4, 64, 1, A) == dq.DQ_ERR_BITS
        assert fn(A, 1, A, A, A + 2, 4, 64, 6, A) == dq.DQ_ERR_ALIGN
        assert fn(A, 1, A, A, A, 4, 64, 6, A + 2) == dq.DQ_ERR_ALIGN


@pytest.mark.parametrize("group", [0, 16, 31, 48, 96, 4096, -32])
def test_group_sizes_rejected(group):
    assert dq.dq_quantize_pack_group(A, dq.DQ_BF16, 4, 64, 6, group, A, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_unpack_group(A, A, 4, 64, 6, group, A, 0) == dq.DQ_ERR_SHAPE
    assert dq.dq_gemv_group(A, 1, A, A, 4, 64, 6, group, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_gemm_group(A, 1, A, A, 4, 64, 6, group, A) == dq.DQ_ERR_SHAPE


def test_group_arguments_rejected():
    assert dq.dq_quantize_pack_group(A, dq.DQ_BF16, 4, 64, 6, 32, A, 0) == dq.DQ_ERR_NULL
    assert dq.dq_quantize_pack_group(A, dq.DQ_BF16, 4, 64, 17, 32, A, A) == dq.DQ_ERR_BITS
    assert dq.dq_quantize_pack_group(A, 5, 4, 64, 6, 32, A, A) == dq.DQ_ERR_DTYPE
    assert dq.dq_quantize_pack_group(A, dq.DQ_BF16, 4, 64, 6, 32, A, A + 1) == dq.DQ_ERR_ALIGN
    assert dq.dq_unpack_group(A, 0, 4, 64, 6, 32, 0, A) == dq.DQ_ERR_NULL
    assert dq.dq_gemv_group(A, 17, A, A, 4, 64, 6, 32, A) == dq.DQ_ERR_SHAPE
    assert dq.dq_gemv_group(MIS, 1, A, A, 4, 64, 6, 32, A) == dq.DQ_ERR_ALIGN
    assert dq.dq_gemm_group(A, 1, A, 0, 4, 64, 6, 32, A) == dq.DQ_ERR_NULL
    assert dq.dq_gemm_group(A, 0, A, A, 4, 64, 6, 32, A) == dq.DQ_ERR_SHAPE


def _items(n, **over):
    arr = (dq.DQGemvItem * n)()
    for i in range(n):
        arr[i] = dq.DQGemvItem(A, A, A, A + 64 * i, 4, 64, 6)
    for k, v in over.items():
        i, field = k.split("_", 1)
        setattr(arr[int(i)], field, v)
    return arr


def test_gemv_batched_arguments_rejected():
    """Every item is checked on the host before anything is enqueued (the fake
    device addresses are never touched)."""
    f = dq.dq_gemv_batched
    addr = ctypes.addressof
    assert f(0, 1, 1) == dq.DQ_ERR_NULL
    assert f(addr(_items(1)), 0, 1) == dq.DQ_ERR_SHAPE
    assert f(addr(_items(33)), 33, 1) == dq.DQ_ERR_SHAPE
    assert f(addr(_items(2)), 2, 0) == dq.DQ_ERR_SHAPE
    assert f(addr(_items(2)), 2, 17) == dq.DQ_ERR_SHAPE
    # a bad last item is found before the good ones run
    for field, value, status in (("x", None, dq.DQ_ERR_NULL), ("packed", None, dq.DQ_ERR_NULL),
                                 ("scales", None, dq.DQ_ERR_NULL), ("y", None, dq.DQ_ERR_NULL),
                                 ("bits", 1, dq.DQ_ERR_BITS), ("bits", 16, dq.DQ_ERR_BITS),
                                 ("N", 0, dq.DQ_ERR_SHAPE), ("K", 0, dq.DQ_ERR_SHAPE),
                                 ("K", (1 << 22) + 1, dq.DQ_ERR_SHAPE), ("N", 1 << 31, dq.DQ_ERR_SHAPE),
                                 ("x", MIS, dq.DQ_ERR_ALIGN), ("packed", MIS, dq.DQ_ERR_ALIGN),
                                 ("scales", A + 2, dq.DQ_ERR_ALIGN), ("y", A + 2, dq.DQ_ERR_ALIGN),
                                 ("group", 16, dq.DQ_ERR_SHAPE), ("group", 96, dq.DQ_ERR_SHAPE),
                                 ("group", 4096, dq.DQ_ERR_SHAPE), ("zeros", A + 2, dq.DQ_ERR_ALIGN)):
        assert f(addr(_items(5, **{"4_" + field: value})), 5, 1) == status, (field, value)
    # zero points and group scales together: no such scheme
    assert f(addr(_items(3, **{"2_group": 64, "2_zeros": A})), 3, 1) == dq.DQ_ERR_SHAPE


def test_gemv_item_layout():
    """dq_gemv_item's fields sit where include/dq.h puts them (the binding's
    ctypes mirror of the struct)."""
    off = {name: getattr(dq.DQGemvItem, name).offset for name, _ in dq.DQGemvItem._fields_}
    assert off == {"x": 0, "packed": 8, "scales": 16, "y": 24, "N": 32, "K": 40, "bits": 48,
                   "group": 52, "zeros": 56}
    assert ctypes.sizeof(dq.DQGemvItem) == 64
