// Host-only driver for the sanitizer pass: the CPU oracle, the host allocator
// (dq_sensitivity, dq_allocate_bits) and the packed-file writer and parser
// (dq_file_*), built with AddressSanitizer and UndefinedBehaviorSanitizer and
// run over random and hostile inputs.  The parser gets thousands of damaged
// files: random byte flips in the header and entry table, offsets and sizes
// near 2^64, truncation.  Whenever dq_file_open accepts a file, every entry's
// regions must lie inside the file (checked here with exact 128-bit sums),
// and reading them (verify, info) must stay in bounds.  Exit status 0 = clean.
#include "../../include/dq.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

extern "C" {
int64_t oracle_row_bytes(int64_t K, int32_t bits);
void oracle_set_threads(int n);
void oracle_quantize_pack(const void* w, int32_t dtype, int64_t N, int64_t K, int32_t bits,
                          uint32_t* packed, float* scales, int32_t* q_out);
void oracle_unpack(const uint32_t* packed, const float* scales, int64_t N, int64_t K, int32_t bits,
                   int32_t* q_out, float* w_out);
void oracle_matmul(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                   int64_t N, int64_t K, int32_t bits, double* y, double* bound);
void oracle_quantize_pack_asym(const void* w, int32_t dtype, int64_t N, int64_t K, int32_t bits,
                               uint32_t* packed, float* scales, int32_t* zeros, uint32_t* u_out);
void oracle_unpack_asym(const uint32_t* packed, const float* scales, const int32_t* zeros,
                        int64_t N, int64_t K, int32_t bits, int32_t* q_out, float* w_out);
void oracle_matmul_asym(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                        const int32_t* zeros, int64_t N, int64_t K, int32_t bits, double* y,
                        double* bound);
void oracle_quantize_pack_group(const void* w, int32_t dtype, int64_t N, int64_t K, int32_t bits,
                                int64_t g, uint32_t* packed, float* scales, int32_t* q_out);
void oracle_unpack_group(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                         int32_t bits, int64_t g, int32_t* q_out, float* w_out);
void oracle_matmul_group(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, int32_t bits, int64_t g, double* y, double* bound);
}

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next()
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}
double uniform() { return (double)(next() >> 11) * 0x1.0p-53; }

int g_fail = 0;
#define EXPECT(cond)                                                                     \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond);                   \
            ++g_fail;                                                                    \
        }                                                                                \
    } while (0)

float special(int i)
{
    const float v[] = {0.0f, -0.0f, NAN, INFINITY, -INFINITY, 1.4e-45f, -3e-39f, 3.4e38f, 1.0f};
    return v[i % 9];
}

void oracle_pass()
{
    const int64_t shapes[][2] = {{1, 1}, {3, 31}, {4, 33}, {2, 300}, {5, 64}};
    for (int bits = 2; bits <= 15; ++bits) {
        for (const auto& sh : shapes) {
            const int64_t N = sh[0], K = sh[1], M = 3;
            std::vector<float> w(N * K);
            for (auto& v : w) v = (float)(uniform() * 2 - 1);
            for (int64_t i = 0; i < N * K; i += 7) w[i] = special((int)(next() % 9));
            std::vector<uint16_t> x(M * K);
            for (auto& v : x) v = (uint16_t)(next() & 0xffff);
            const int64_t rw = oracle_row_bytes(K, bits) / 4;
            std::vector<uint32_t> packed(N * rw);
            std::vector<float> s(N), wo(N * K);
            std::vector<int32_t> q(N * K), z(N);
            std::vector<uint32_t> u(N * K);
            std::vector<double> y(M * N), b(M * N);
            oracle_quantize_pack(w.data(), 0, N, K, bits, packed.data(), s.data(), q.data());
            oracle_unpack(packed.data(), s.data(), N, K, bits, q.data(), wo.data());
            oracle_matmul(x.data(), M, packed.data(), s.data(), N, K, bits, y.data(), b.data());
            oracle_quantize_pack_asym(w.data(), 0, N, K, bits, packed.data(), s.data(), z.data(),
                                      u.data());
            oracle_unpack_asym(packed.data(), s.data(), z.data(), N, K, bits, q.data(), wo.data());
            oracle_matmul_asym(x.data(), M, packed.data(), s.data(), z.data(), N, K, bits, y.data(),
                               b.data());
            for (int64_t g : {32, 64, 2048}) {
                const int64_t G = (K + g - 1) / g;
                std::vector<float> sg(N * G);
                oracle_quantize_pack_group(w.data(), 0, N, K, bits, g, packed.data(), sg.data(),
                                           q.data());
                oracle_unpack_group(packed.data(), sg.data(), N, K, bits, g, q.data(), wo.data());
                oracle_matmul_group(x.data(), M, packed.data(), sg.data(), N, K, bits, g, y.data(),
                                    b.data());
            }
        }
    }
}

void recipe_pass()
{
    const int32_t native[] = {4, 8, 16};
    int32_t full[13];
    for (int i = 0; i < 13; ++i) full[i] = 4 + i;
    for (int it = 0; it < 400; ++it) {
        const int64_t n = 1 + (int64_t)(next() % 60);
        std::vector<double> h(n), ss(n), sens(n);
        std::vector<int64_t> params(n);
        for (int64_t i = 0; i < n; ++i) {
            h[i] = (next() % 7 == 0) ? 0.0 : std::exp(uniform() * 8 - 4);
            params[i] = 1 + (int64_t)(next() % (it % 5 == 0 ? (uint64_t)DQ_MAX_PARAMS : 100000));
            ss[i] = uniform() * (double)params[i];
        }
        EXPECT(dq_sensitivity(h.data(), ss.data(), params.data(), n, sens.data()) == DQ_OK);
        const bool nat = it % 2;
        const int32_t* lv = nat ? native : full;
        const int32_t nl = nat ? 3 : 13;
        double floor_bits = 0;
        for (int64_t i = 0; i < n; ++i) floor_bits += (double)params[i] * lv[0];
        const int64_t budgets[] = {-1, (int64_t)floor_bits, (int64_t)(floor_bits * 1.4),
                                   (int64_t)floor_bits - 1};
        for (int64_t budget : budgets) {
            std::vector<int32_t> bits(n);
            const int64_t cap = (int64_t)(next() % 3 == 0 ? 0 : next() % 2000);
            std::vector<int64_t> sm(cap > 0 ? cap : 1);
            std::vector<int32_t> sb(cap > 0 ? cap : 1);
            int64_t steps = 0;
            double loss = 0;
            const dq_status st =
                dq_allocate_bits(sens.data(), params.data(), n, lv, nl, budget, bits.data(),
                                 cap ? sm.data() : nullptr, cap ? sb.data() : nullptr, cap, &steps,
                                 &loss);
            EXPECT(st == DQ_OK || st == DQ_ERR_BUDGET);
            if (st == DQ_OK)
                for (int64_t i = 0; i < n; ++i) EXPECT(bits[i] >= lv[0] && bits[i] <= 16);
        }
    }
    // hostile arguments: each must be refused, not crash
    double bad_s[2] = {NAN, 1.0}, ok_s[2] = {1.0, 2.0};
    int64_t p2[2] = {10, 10}, bad_p[2] = {0, 10};
    int32_t out[2];
    const int32_t bad_lv[] = {8, 4};
    EXPECT(dq_allocate_bits(bad_s, p2, 2, native, 3, -1, out, nullptr, nullptr, 0, nullptr,
                            nullptr) != DQ_OK);
    EXPECT(dq_allocate_bits(ok_s, bad_p, 2, native, 3, -1, out, nullptr, nullptr, 0, nullptr,
                            nullptr) != DQ_OK);
    EXPECT(dq_allocate_bits(ok_s, p2, 2, bad_lv, 2, -1, out, nullptr, nullptr, 0, nullptr,
                            nullptr) != DQ_OK);
    EXPECT(dq_sensitivity(bad_s, ok_s, p2, 2, out ? ok_s : nullptr) != DQ_OK);
}

void put_u64(std::vector<unsigned char>& b, size_t off, uint64_t v)
{
    for (int i = 0; i < 8; ++i) b[off + i] = (unsigned char)(v >> (8 * i));
}
uint64_t get_u64(const std::vector<unsigned char>& b, size_t off)
{
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i) v |= (uint64_t)b[off + i] << (8 * i);
    return v;
}

std::vector<unsigned char> read_file(const std::string& p)
{
    std::vector<unsigned char> b;
    FILE* f = std::fopen(p.c_str(), "rb");
    if (!f) return b;
    unsigned char buf[65536];
    size_t n;
    while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) b.insert(b.end(), buf, buf + n);
    std::fclose(f);
    return b;
}

void write_file(const std::string& p, const std::vector<unsigned char>& b, size_t len)
{
    FILE* f = std::fopen(p.c_str(), "wb");
    if (!f) return;
    if (len) std::fwrite(b.data(), 1, len, f);
    std::fclose(f);
}

// open a (possibly damaged) file image; if accepted, every region must lie in
// the file and reading it must stay in bounds
void probe(const std::string& path, const std::vector<unsigned char>& img, size_t len)
{
    write_file(path, img, len);
    dq_file* f = nullptr;
    const dq_status st = dq_file_open(path.c_str(), &f);
    if (st != DQ_OK) {
        EXPECT(f == nullptr);
        return;
    }
    const int64_t count = dq_file_count(f);
    for (int64_t i = 0; i < count; ++i) {
        const size_t e = 64 + 128 * (size_t)i;
        const uint64_t doff = get_u64(img, e + 88), db = get_u64(img, e + 96);
        const uint64_t soff = get_u64(img, e + 104);
        dq_file_matrix m;
        EXPECT(dq_file_matrix_info(f, i, &m) == DQ_OK);
        const uint64_t sb = soff ? (uint64_t)m.N * 4 : 0;
        EXPECT((unsigned __int128)doff + db <= len);
        EXPECT((unsigned __int128)soff + sb <= len);
        (void)dq_file_verify(f, i);
    }
    dq_file_close(f);
}

void packfile_pass(const std::string& dir)
{
    const std::string path = dir + "/sanitize.dqw";
    std::vector<std::vector<uint32_t>> data;
    std::vector<std::vector<float>> scales;
    std::vector<dq_file_matrix> mats;
    // regions below and above 4096 bytes (an offset 2^64 - 4096 k wraps only
    // when the region is at least 4096 k bytes)
    const int64_t shapes[][3] = {{3, 40, 5}, {2, 33, 16}, {32, 32, 2}, {40, 300, 7}, {4, 100, 15}};
    for (const auto& sh : shapes) {
        dq_file_matrix m;
        std::memset(&m, 0, sizeof m);
        std::snprintf(m.name, sizeof m.name, "m%lld", (long long)sh[2]);
        m.N = sh[0];
        m.K = sh[1];
        m.bits = (int32_t)sh[2];
        const size_t words =
            m.bits == 16 ? (size_t)(m.N * m.K + 1) / 2 : (size_t)(m.N * oracle_row_bytes(m.K, m.bits) / 4);
        data.emplace_back(words);
        for (auto& v : data.back()) v = (uint32_t)next();
        scales.emplace_back(m.bits == 16 ? 0 : m.N);
        for (auto& v : scales.back()) v = (float)uniform();
        mats.push_back(m);
    }
    for (size_t i = 0; i < mats.size(); ++i) {
        mats[i].data = data[i].data();
        mats[i].scales = mats[i].bits == 16 ? nullptr : scales[i].data();
    }
    EXPECT(dq_file_write(path.c_str(), mats.data(), (int64_t)mats.size()) == DQ_OK);
    const std::vector<unsigned char> good = read_file(path);
    EXPECT(good.size() > 64);
    probe(path, good, good.size());
    const size_t table_end = 64 + 128 * mats.size();
    const uint64_t nasty[] = {~0ull, 0ull - 4096, 0ull - 4096 * 2, 0ull - 4096 * 3,
                              0ull - 4096 * 4, ~0ull - 4096 * 2 + 1, 1ull << 63,
                              (1ull << 63) - 4096, good.size(), good.size() - 4096,
                              good.size() + 4096, 0};
    constexpr uint64_t kNasty = sizeof nasty / sizeof nasty[0];
    for (int it = 0; it < 6000; ++it) {
        std::vector<unsigned char> img = good;
        size_t len = img.size();
        switch (it % 4) {
        case 0:  // random byte flips in the header and table
            for (int k = 0; k < 1 + (int)(next() % 4); ++k)
                img[next() % table_end] ^= (unsigned char)(1u << (next() % 8));
            break;
        case 1: {  // a field of one entry set to a hostile value
            const size_t e = 64 + 128 * (next() % mats.size());
            const size_t fields[] = {64, 72, 88, 96, 104};
            put_u64(img, e + fields[next() % 5], nasty[next() % kNasty]);
            break;
        }
        case 2:  // header count / table / size fields
            put_u64(img, 16 + 8 * (next() % 2), nasty[next() % kNasty]);
            if (next() % 2) img[12] = (unsigned char)next();
            break;
        default:  // truncation
            len = (size_t)(next() % img.size());
            break;
        }
        probe(path, img, len);
    }
}

}  // namespace

int main(int argc, char** argv)
{
    const std::string dir = argc > 1 ? argv[1] : ".";
    oracle_set_threads(1);
    oracle_pass();
    recipe_pass();
    packfile_pass(dir);
    std::printf("sanitize driver: %d failures\n", g_fail);
    return g_fail ? 1 : 0;
}
