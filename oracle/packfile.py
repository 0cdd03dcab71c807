"""CPU oracle for the on-disk packed-weight format: an independent writer and
reader of the layout, written from its specification with ``struct``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``.  The product package never
imports it and shares no code with it.

Source: DynaQuant page (zingnex.cn), "项目现状与路线图" (an on-disk format for
packed weights is listed as in progress); the layout itself is the library's
own, specified in its C header:

* header (64 bytes): b"DQWPACK1", u32 version 1, u32 count, u64 table offset
  64, u64 file size, 32 zero bytes;
* count entries of 128 bytes: name (64 bytes, UTF-8, NUL-padded), i64 N,
  i64 K, i32 bits, u32 flags 0, u64 data offset, u64 data bytes, u64 scales
  offset (0 if none), u64 checksum, u64 0;
* regions in entry order, each at a multiple of 4096, zero bytes between and
  after the last one up to the next multiple of 4096: bits 2..15 -- the packed
  words [N, row_words] then fp32 scales [N]; bits 16 -- bf16 [N, K], no scales;
* checksum: 64-bit FNV-1a over the data bytes then the scale bytes.
All integers little-endian.
"""
from __future__ import annotations

import struct

MAGIC = b"DQWPACK1"
ALIGN = 4096
HEADER = struct.Struct("<8sIIQQ32s")
ENTRY = struct.Struct("<64sqqiIQQQQQ")
FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for byte in data:
        h = ((h ^ byte) * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def row_bytes(K: int, bits: int) -> int:
    return (-(-K * bits // 8) + 127) // 128 * 128


def region_sizes(N: int, K: int, bits: int):
    if bits == 16:
        return N * K * 2, 0
    if not 2 <= bits <= 15:
        raise ValueError("bits")
    return N * row_bytes(K, bits), N * 4


def _up(v: int) -> int:
    return -(-v // ALIGN) * ALIGN


def write_bytes(matrices) -> bytes:
    """matrices: (name, N, K, bits, data bytes, scale bytes or b"")."""
    count = len(matrices)
    off = _up(HEADER.size + ENTRY.size * count)
    entries, regions = [], []
    for name, N, K, bits, data, scales in matrices:
        db, sb = region_sizes(N, K, bits)
        assert len(data) == db and len(scales) == sb
        doff = off
        soff = _up(doff + db) if sb else 0
        off = _up(soff + sb if sb else doff + db)
        entries.append(ENTRY.pack(name.encode("utf-8"), N, K, bits, 0, doff, db, soff,
                                  fnv1a64(scales, fnv1a64(data)), 0))
        regions.append((doff, data))
        if sb:
            regions.append((soff, scales))
    out = bytearray(off)
    out[:HEADER.size] = HEADER.pack(MAGIC, 1, count, HEADER.size, off, b"\0" * 32)
    for i, e in enumerate(entries):
        at = HEADER.size + ENTRY.size * i
        out[at:at + ENTRY.size] = e
    for at, blob in regions:
        out[at:at + len(blob)] = blob
    return bytes(out)


def read_bytes(blob: bytes):
    """Parse a file's bytes; raises ValueError on anything the layout forbids.
    Returns a list of (name, N, K, bits, data bytes, scale bytes, checksum_ok)."""
    if len(blob) < HEADER.size:
        raise ValueError("short file")
    magic, version, count, table, size, pad = HEADER.unpack_from(blob, 0)
    if magic != MAGIC or version != 1 or table != HEADER.size or size != len(blob):
        raise ValueError("bad header")
    if count < 1 or HEADER.size + ENTRY.size * count > len(blob):
        raise ValueError("bad count")
    out, prev = [], HEADER.size + ENTRY.size * count
    for i in range(count):
        (name, N, K, bits, flags, doff, db, soff, csum, _res) = ENTRY.unpack_from(
            blob, HEADER.size + ENTRY.size * i)
        if b"\0" not in name or flags != 0:
            raise ValueError("bad entry %d" % i)
        if not (1 <= N <= 2 ** 31 - 1 and 1 <= K <= 2 ** 22):
            raise ValueError("bad shape %d" % i)
        want_db, sb = region_sizes(N, K, bits)
        if db != want_db or doff % ALIGN or doff < prev or doff + db > len(blob):
            raise ValueError("bad data region %d" % i)
        prev = doff + db
        if sb:
            if soff % ALIGN or soff < prev or soff + sb > len(blob):
                raise ValueError("bad scales region %d" % i)
            prev = soff + sb
        elif soff != 0:
            raise ValueError("scales for bits 16 %d" % i)
        data = blob[doff:doff + db]
        scales = blob[soff:soff + sb] if sb else b""
        out.append((name.split(b"\0", 1)[0].decode("utf-8"), N, K, bits, data, scales,
                    fnv1a64(scales, fnv1a64(data)) == csum))
    return out
