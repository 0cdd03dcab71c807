// On-disk packed-weight format: a recipe's packed matrices, their scales and
// their widths in one file that maps straight into memory (DynaQuant page,
// "项目现状与路线图": a packed-weight storage format on disk is listed as work in
// progress; the layout below is this library's own).
//
// File layout (all integers little-endian):
//   [0, 64)     header: magic "DQWPACK1", u32 version (1), u32 count,
//               u64 table offset (64), u64 file bytes, 32 reserved zero bytes
//   [64, 64 + 128 * count)  one entry per matrix:
//               char name[64] (UTF-8, NUL-padded), i64 N, i64 K, i32 bits,
//               u32 flags (0), u64 data offset, u64 data bytes, u64 scales
//               offset, u64 checksum, u64 reserved (0)
//   data        for 2 <= bits <= 15: the packed words exactly as in device
//               memory, [N, row_words] (row pitch dq_packed_row_bytes(K, bits));
//               for bits == 16 (BF16 weights kept): [N, K] bf16; then fp32
//               scales [N] (none for bits == 16).  Every region starts at a
//               multiple of 4096 bytes, in entry order, zero bytes between.
//   checksum    64-bit FNV-1a over the data bytes then the scale bytes:
//               h = 0xcbf29ce484222325; for each byte: h = (h ^ byte) * 0x100000001b3
//               (mod 2^64).
// This file is host-only C++ (no HIP): the copy of an entry to the device,
// dq_file_load, sits with the other HIP entry points in api.cpp.
#include "../../include/dq.h"

#include <cstdio>
#include <cstring>
#include <new>

#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include "layout.hpp"

namespace {

constexpr char kMagic[8] = {'D', 'Q', 'W', 'P', 'A', 'C', 'K', '1'};
constexpr uint32_t kVersion = 1;
constexpr uint64_t kHeaderBytes = 64;
constexpr uint64_t kEntryBytes = 128;
constexpr uint64_t kAlign = 4096;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

void put_u32(unsigned char* p, uint32_t v)
{
    for (int i = 0; i < 4; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
void put_u64(unsigned char* p, uint64_t v)
{
    for (int i = 0; i < 8; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
uint32_t get_u32(const unsigned char* p)
{
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
    return v;
}
uint64_t get_u64(const unsigned char* p)
{
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
    return v;
}

// 64-bit FNV-1a over a byte stream (fed in pieces).
struct Hash {
    uint64_t h = 0xcbf29ce484222325ull;
    void bytes(const unsigned char* p, uint64_t n)
    {
        uint64_t v = h;
        for (uint64_t i = 0; i < n; ++i) v = (v ^ p[i]) * 0x100000001b3ull;
        h = v;
    }
    uint64_t done() const { return h; }
};

// Sizes of one matrix's regions; false if the description is out of range.
bool region_bytes(int64_t N, int64_t K, int32_t bits, uint64_t* data, uint64_t* scales)
{
    if (N < 1 || N > 0x7fffffffLL || K < 1 || K > DQ_MAX_K) return false;
    if (bits == DQ_TOP_BITS) {
        *data = (uint64_t)N * (uint64_t)K * 2;
        *scales = 0;
        return true;
    }
    if (bits < DQ_MIN_BITS || bits > DQ_MAX_BITS) return false;
    *data = (uint64_t)N * (uint64_t)dq::packed_row_words(K, bits) * 4;
    *scales = (uint64_t)N * 4;
    return true;
}

bool write_all(int fd, const void* p, uint64_t n)
{
    const unsigned char* c = static_cast<const unsigned char*>(p);
    while (n > 0) {
        const ssize_t w = ::write(fd, c, n > (1u << 30) ? (1u << 30) : (size_t)n);
        if (w <= 0) return false;
        c += w;
        n -= (uint64_t)w;
    }
    return true;
}

bool write_zeros(int fd, uint64_t n)
{
    static const unsigned char z[4096] = {};
    while (n > 0) {
        const uint64_t k = n > sizeof z ? sizeof z : n;
        if (!write_all(fd, z, k)) return false;
        n -= k;
    }
    return true;
}

}  // namespace

struct dq_file {
    const unsigned char* base = nullptr;
    uint64_t bytes = 0;
    int64_t count = 0;
};

extern "C" {

dq_status dq_file_write(const char* path, const dq_file_matrix* mats, int64_t count)
{
    if (!path || !mats) return DQ_ERR_NULL;
    if (count < 1 || count > DQ_FILE_MAX_MATRICES) return DQ_ERR_SHAPE;
    // lay out every region and check every description before touching the file
    const uint64_t table_end = kHeaderBytes + kEntryBytes * (uint64_t)count;
    uint64_t off = align_up(table_end);
    unsigned char* table = new (std::nothrow) unsigned char[table_end];
    if (!table) return DQ_ERR_IO;
    std::memset(table, 0, table_end);
    for (int64_t i = 0; i < count; ++i) {
        const dq_file_matrix& m = mats[i];
        uint64_t db, sb;
        if (!region_bytes(m.N, m.K, m.bits, &db, &sb)) {
            delete[] table;
            return m.bits == DQ_TOP_BITS || (m.bits >= DQ_MIN_BITS && m.bits <= DQ_MAX_BITS)
                       ? DQ_ERR_SHAPE
                       : DQ_ERR_BITS;
        }
        if (!m.data || (sb > 0 && !m.scales)) {
            delete[] table;
            return DQ_ERR_NULL;
        }
        if (memchr(m.name, 0, sizeof m.name) == nullptr) {  // names are NUL-terminated
            delete[] table;
            return DQ_ERR_VALUE;
        }
        Hash h;
        h.bytes(static_cast<const unsigned char*>(m.data), db);
        if (sb > 0) h.bytes(reinterpret_cast<const unsigned char*>(m.scales), sb);
        unsigned char* e = table + kHeaderBytes + kEntryBytes * (uint64_t)i;
        const size_t nlen = strnlen(m.name, sizeof m.name);
        std::memcpy(e, m.name, nlen);
        put_u64(e + 64, (uint64_t)m.N);
        put_u64(e + 72, (uint64_t)m.K);
        put_u32(e + 80, (uint32_t)m.bits);
        put_u32(e + 84, 0);
        put_u64(e + 88, off);
        put_u64(e + 96, db);
        const uint64_t soff = sb > 0 ? align_up(off + db) : 0;
        put_u64(e + 104, soff);
        put_u64(e + 112, h.done());
        off = align_up(sb > 0 ? soff + sb : off + db);
    }
    std::memcpy(table, kMagic, 8);
    put_u32(table + 8, kVersion);
    put_u32(table + 12, (uint32_t)count);
    put_u64(table + 16, kHeaderBytes);
    put_u64(table + 24, off);

    const int fd = ::open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) {
        delete[] table;
        return DQ_ERR_IO;
    }
    bool ok = write_all(fd, table, table_end);
    uint64_t pos = table_end;
    for (int64_t i = 0; ok && i < count; ++i) {
        const unsigned char* e = table + kHeaderBytes + kEntryBytes * (uint64_t)i;
        const uint64_t doff = get_u64(e + 88), db = get_u64(e + 96), soff = get_u64(e + 104);
        ok = write_zeros(fd, doff - pos) && write_all(fd, mats[i].data, db);
        pos = doff + db;
        if (ok && soff > 0) {
            const uint64_t sb = (uint64_t)mats[i].N * 4;
            ok = write_zeros(fd, soff - pos) && write_all(fd, mats[i].scales, sb);
            pos = soff + sb;
        }
    }
    const uint64_t total = get_u64(table + 24);
    ok = ok && write_zeros(fd, total - pos);
    delete[] table;
    if (::close(fd) != 0) ok = false;
    return ok ? DQ_OK : DQ_ERR_IO;
}

dq_status dq_file_open(const char* path, dq_file** out)
{
    if (!path || !out) return DQ_ERR_NULL;
    *out = nullptr;
    const int fd = ::open(path, O_RDONLY);
    if (fd < 0) return DQ_ERR_IO;
    struct stat st;
    if (fstat(fd, &st) != 0) {
        ::close(fd);
        return DQ_ERR_IO;
    }
    const uint64_t size = (uint64_t)st.st_size;
    if (size < kHeaderBytes) {
        ::close(fd);
        return DQ_ERR_FORMAT;
    }
    void* map = mmap(nullptr, size, PROT_READ, MAP_SHARED, fd, 0);
    ::close(fd);
    if (map == MAP_FAILED) return DQ_ERR_IO;
    const unsigned char* b = static_cast<const unsigned char*>(map);
    // the header and every entry must describe regions inside the file, in order
    bool ok = std::memcmp(b, kMagic, 8) == 0 && get_u32(b + 8) == kVersion &&
              get_u64(b + 16) == kHeaderBytes && get_u64(b + 24) == size;
    const uint64_t count = ok ? get_u32(b + 12) : 0;
    ok = ok && count >= 1 && count <= (uint64_t)DQ_FILE_MAX_MATRICES &&
         kHeaderBytes + kEntryBytes * count <= size;
    uint64_t prev_end = kHeaderBytes + kEntryBytes * count;
    for (uint64_t i = 0; ok && i < count; ++i) {
        const unsigned char* e = b + kHeaderBytes + kEntryBytes * i;
        const int64_t N = (int64_t)get_u64(e + 64), K = (int64_t)get_u64(e + 72);
        const int32_t bits = (int32_t)get_u32(e + 80);
        uint64_t db, sb;
        ok = memchr(e, 0, 64) != nullptr && get_u32(e + 84) == 0 &&
             region_bytes(N, K, bits, &db, &sb);
        if (!ok) break;
        const uint64_t doff = get_u64(e + 88), soff = get_u64(e + 104);
        // offsets are untrusted: compare without forming doff + db (which
        // could wrap past 2^64 and pass)
        ok = get_u64(e + 96) == db && doff % kAlign == 0 && doff >= prev_end && doff <= size &&
             db <= size - doff;
        prev_end = ok ? doff + db : prev_end;
        if (ok && sb > 0) {
            ok = soff % kAlign == 0 && soff >= prev_end && soff <= size && sb <= size - soff;
            prev_end = ok ? soff + sb : prev_end;
        } else if (ok) {
            ok = soff == 0;
        }
    }
    if (!ok) {
        munmap(map, size);
        return DQ_ERR_FORMAT;
    }
    dq_file* f = new (std::nothrow) dq_file;
    if (!f) {
        munmap(map, size);
        return DQ_ERR_IO;
    }
    f->base = b;
    f->bytes = size;
    f->count = (int64_t)count;
    *out = f;
    return DQ_OK;
}

int64_t dq_file_count(const dq_file* f) { return f ? f->count : 0; }

dq_status dq_file_matrix_info(const dq_file* f, int64_t i, dq_file_matrix* out)
{
    if (!f || !out) return DQ_ERR_NULL;
    if (i < 0 || i >= f->count) return DQ_ERR_SHAPE;
    const unsigned char* e = f->base + kHeaderBytes + kEntryBytes * (uint64_t)i;
    std::memset(out, 0, sizeof *out);
    std::memcpy(out->name, e, 64);
    out->N = (int64_t)get_u64(e + 64);
    out->K = (int64_t)get_u64(e + 72);
    out->bits = (int32_t)get_u32(e + 80);
    out->data = f->base + get_u64(e + 88);
    const uint64_t soff = get_u64(e + 104);
    out->scales = soff ? reinterpret_cast<const float*>(f->base + soff) : nullptr;
    return DQ_OK;
}

dq_status dq_file_verify(const dq_file* f, int64_t i)
{
    if (!f) return DQ_ERR_NULL;
    if (i < 0 || i >= f->count) return DQ_ERR_SHAPE;
    const unsigned char* e = f->base + kHeaderBytes + kEntryBytes * (uint64_t)i;
    Hash h;
    h.bytes(f->base + get_u64(e + 88), get_u64(e + 96));
    const uint64_t soff = get_u64(e + 104);
    if (soff) h.bytes(f->base + soff, get_u64(e + 64) * 4);
    return h.done() == get_u64(e + 112) ? DQ_OK : DQ_ERR_FORMAT;
}

void dq_file_close(dq_file* f)
{
    if (!f) return;
    munmap(const_cast<unsigned char*>(f->base), f->bytes);
    delete f;
}

}  // extern "C"
