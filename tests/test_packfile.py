"""The on-disk packed-weight format (CPU only): the oracle writer/reader
against a file laid out by hand and FNV-1a's published vectors, then the
library's dq_file_* calls against the oracle byte for byte, and every way a
file or a description can be refused.

Source: DynaQuant page (zingnex.cn), "项目现状与路线图" (packed-weight format
on disk, in progress); the layout is the library's own (include/dq.h)."""
from __future__ import annotations

import ctypes
import os
import struct

import numpy as np
import pytest

import mixed_precision_weight_dq_amd as dq
from oracle import packfile as opf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "packfile_example.txt")


def golden_lines():
    out = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].split()
        if line:
            out.append((int(line[0]), bytes(int(h, 16) for h in line[1:])))
    return out


def example_matrix():
    rng = np.random.default_rng(1)
    data = rng.integers(0, 2 ** 32, (2, 32), dtype=np.uint32)
    scales = np.array([0.25, 3.5], dtype=np.float32)
    return ("w0", 2, 3, 5, data, scales)


def test_fnv1a64_published_vectors():
    assert opf.fnv1a64(b"") == 0xCBF29CE484222325
    assert opf.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert opf.fnv1a64(b"foobar") == 0x85944171F73967E8
    # feeding in pieces continues the same stream
    assert opf.fnv1a64(b"bar", opf.fnv1a64(b"foo")) == opf.fnv1a64(b"foobar")


def test_oracle_writer_matches_hand_layout():
    name, N, K, bits, data, scales = example_matrix()
    blob = opf.write_bytes([(name, N, K, bits, data.tobytes(), scales.tobytes())])
    assert len(blob) == 12288
    for off, want in golden_lines():
        assert blob[off:off + len(want)] == want, "offset %d" % off
    assert blob[4096:4096 + 256] == data.tobytes()
    assert blob[8192:8200] == scales.tobytes()
    assert struct.unpack_from("<Q", blob, 176)[0] == opf.fnv1a64(data.tobytes() + scales.tobytes())
    # every other byte is zero
    mask = np.ones(len(blob), bool)
    for off, want in golden_lines():
        mask[off:off + len(want)] = False
    mask[176:184] = False
    mask[66:128] = False  # the name's NUL padding, checked below
    mask[4096:4096 + 256] = False
    mask[8192:8200] = False
    assert not np.frombuffer(blob, np.uint8)[mask].any()
    assert blob[66:128] == b"\0" * 62
    (got,) = opf.read_bytes(blob)
    assert got[:4] == (name, N, K, bits) and got[4] == data.tobytes() and got[6]


def random_set(seed: int):
    rng = np.random.default_rng(seed)
    mats = []
    for i, bits in enumerate([2, 5, 6, 9, 15, 16, 8, 4]):
        N = int(rng.integers(1, 40))
        K = int(rng.integers(1, 700))
        if bits == 16:
            data = rng.integers(0, 2 ** 16, (N, K), dtype=np.uint16)
            scales = None
        else:
            data = rng.integers(0, 2 ** 32, (N, dq.dq_packed_row_bytes(K, bits) // 4), dtype=np.uint32)
            scales = rng.standard_normal(N).astype(np.float32)
        mats.append(("layer%d.%s" % (i, "gewicht-ß" if i % 2 else "w"), N, K, bits, data, scales))
    return mats


def as_oracle(mats):
    return [(n, N, K, b, d.tobytes(), s.tobytes() if s is not None else b"")
            for n, N, K, b, d, s in mats]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_writes_the_oracle_bytes(tmp_path, seed):
    mats = random_set(seed)
    path = str(tmp_path / "set.dqw")
    dq.write_packed_file(path, mats)
    with open(path, "rb") as f:
        blob = f.read()
    assert blob == opf.write_bytes(as_oracle(mats))


def test_library_reads_oracle_files(tmp_path):
    mats = random_set(7) + [example_matrix()]
    path = str(tmp_path / "o.dqw")
    with open(path, "wb") as f:
        f.write(opf.write_bytes(as_oracle(mats)))
    with dq.PackedFile(path) as pf:
        assert len(pf) == len(mats)
        for i, (n, N, K, b, d, s) in enumerate(mats):
            name, N2, K2, b2, data, scales = pf.info(i)
            assert (name, N2, K2, b2) == (n, N, K, b)
            assert data.tobytes() == d.tobytes()
            assert (scales is None) == (s is None)
            if s is not None:
                assert scales.tobytes() == s.tobytes()
            assert pf.verify(i)


def test_corruption_and_bad_files_refused(tmp_path):
    mats = random_set(3)
    good = bytearray(opf.write_bytes(as_oracle(mats)))

    def opens(blob):
        p = str(tmp_path / "x.dqw")
        with open(p, "wb") as f:
            f.write(bytes(blob))
        try:
            with dq.PackedFile(p) as pf:
                return [pf.verify(i) for i in range(len(pf))]
        except dq.DQError as e:
            return e.status

    assert all(opens(good))
    # one flipped data byte: the file opens, that entry fails its checksum
    bad = bytearray(good)
    doff = struct.unpack_from("<Q", good, 64 + 88)[0]
    bad[doff + 3] ^= 0x10
    assert opens(bad) == [False] + [True] * (len(mats) - 1)
    with pytest.raises(ValueError):
        opf.read_bytes(bytes(bad)[:-1])
    assert not opf.read_bytes(bytes(bad))[0][6]
    # header and entry damage
    cases = {
        "magic": (0, b"DQWPACK2"),
        "version": (8, struct.pack("<I", 2)),
        "count0": (12, struct.pack("<I", 0)),
        "table": (16, struct.pack("<Q", 128)),
        "size": (24, struct.pack("<Q", len(good) + 4096)),
        "flags": (64 + 84, struct.pack("<I", 1)),
        "bits": (64 + 80, struct.pack("<i", 17)),
        "N0": (64 + 64, struct.pack("<q", 0)),
        "data_bytes": (64 + 96, struct.pack("<Q", 4)),
        "misaligned": (64 + 88, struct.pack("<Q", doff + 8)),
        "overlap": (64 + 128 + 88, struct.pack("<Q", doff)),
        "name_no_nul": (64, b"n" * 64),
        # offsets near 2^64: offset + size wraps to a small number, which a
        # check that adds them would let through
        "data_offset_wraps": (64 + 88, struct.pack("<Q", 2 ** 64 - 4096)),
        "scale_offset_wraps": (64 + 104, struct.pack("<Q", 2 ** 64 - 4096)),
        "last_data_offset_wraps": (64 + 128 * (len(mats) - 1) + 88,
                                   struct.pack("<Q", 2 ** 64 - 4096)),
    }
    for what, (off, patch) in cases.items():
        blob = bytearray(good)
        blob[off:off + len(patch)] = patch
        assert opens(blob) == dq.DQ_ERR_FORMAT, what
        with pytest.raises(ValueError):
            opf.read_bytes(bytes(blob))
    assert opens(good[:-4096]) == dq.DQ_ERR_FORMAT  # truncated
    assert opens(good[:10]) == dq.DQ_ERR_FORMAT


def test_write_arguments_refused(tmp_path):
    lib = dq.load()
    arr = (dq.DQFileMatrix * 1)()
    data = np.zeros((2, 32), np.uint32)
    scales = np.zeros(2, np.float32)
    arr[0].name = b"m"
    arr[0].N, arr[0].K, arr[0].bits = 2, 3, 5
    arr[0].data, arr[0].scales = data.ctypes.data, scales.ctypes.data
    p = str(tmp_path / "w.dqw").encode()
    assert lib.dq_file_write(p, arr, 1) == dq.DQ_OK
    assert lib.dq_file_write(None, arr, 1) == dq.DQ_ERR_NULL
    assert lib.dq_file_write(p, arr, 0) == dq.DQ_ERR_SHAPE
    for field, value, status in (("bits", 17, dq.DQ_ERR_BITS), ("bits", 1, dq.DQ_ERR_BITS),
                                 ("N", 0, dq.DQ_ERR_SHAPE), ("K", (1 << 22) + 1, dq.DQ_ERR_SHAPE),
                                 ("data", None, dq.DQ_ERR_NULL), ("scales", None, dq.DQ_ERR_NULL)):
        old = getattr(arr[0], field)
        setattr(arr[0], field, value)
        assert lib.dq_file_write(p, arr, 1) == status, field
        setattr(arr[0], field, old)
    arr[0].name = b"n" * 63
    assert lib.dq_file_write(p, arr, 1) == dq.DQ_OK
    ctypes.memmove(ctypes.addressof(arr[0]), b"n" * 64, 64)  # no NUL in the 64 bytes
    assert lib.dq_file_write(p, arr, 1) == dq.DQ_ERR_VALUE
    assert lib.dq_file_write(str(tmp_path / "no" / "dir.dqw").encode(), (dq.DQFileMatrix * 1)(
        dq.DQFileMatrix(b"m", 2, 3, 5, data.ctypes.data, scales.ctypes.data)), 1) == dq.DQ_ERR_IO
    with pytest.raises(dq.DQError) as e:
        dq.PackedFile(str(tmp_path / "missing.dqw"))
    assert e.value.status == dq.DQ_ERR_IO
    assert lib.dq_file_count(None) == 0
    lib.dq_file_close(None)


def test_load_arguments_refused(tmp_path):
    """dq_file_load checks its arguments on the host before any HIP call (the
    fake device addresses are never touched)."""
    A = 1 << 20
    p = str(tmp_path / "l.dqw")
    dq.write_packed_file(p, random_set(4))
    lib = dq.load()
    with dq.PackedFile(p) as pf:
        h = pf._h
        assert lib.dq_file_load(h, 0, 0, A, 0) == dq.DQ_ERR_NULL
        assert lib.dq_file_load(h, 0, A, 0, 0) == dq.DQ_ERR_NULL  # this entry has scales
        assert lib.dq_file_load(h, 0, A + 4, A, 0) == dq.DQ_ERR_ALIGN
        assert lib.dq_file_load(h, 0, A, A + 2, 0) == dq.DQ_ERR_ALIGN
        assert lib.dq_file_load(h, -1, A, A, 0) == dq.DQ_ERR_SHAPE
        assert lib.dq_file_load(h, len(pf), A, A, 0) == dq.DQ_ERR_SHAPE
        assert lib.dq_file_load(None, 0, A, A, 0) == dq.DQ_ERR_NULL
        assert lib.dq_file_verify(h, len(pf)) == dq.DQ_ERR_SHAPE
        assert lib.dq_file_matrix_info(h, len(pf), ctypes.byref(dq.DQFileMatrix())) == dq.DQ_ERR_SHAPE
