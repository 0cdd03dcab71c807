// Host-side brute-force check of the quantizer's rounded quotient
// (rounded_quotient in quant_rule.hpp, the function the quantize kernels
// inline): for every width b = 2 .. 15, both schemes' limits (qmax + 1 and
// L + 1), and row maxima across the fp32 range -- including maxima whose scale
// has a subnormal reciprocal (b = 2, 3 near the top of the range) and tiny
// maxima whose reciprocal overflows -- every w within 6 ulps of each rounding
// tie (j + 1/2) s and of each level j s, plus random w, must round to
// rint(fl32(w / s)) exactly as the IEEE divide does.  Runs on the CPU only.
#include "../../mixed_precision_weight_dq_amd/csrc/quant_rule.hpp"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

namespace {

uint64_t g_checked = 0, g_fast = 0, g_bad = 0, g_rand = 0, g_rand_fast = 0;

void check(float w, float s, float r, float margin, float amax, bool random = false)
{
    if (!(std::fabs(w) <= amax)) return;  // the rule's premise: |w| <= the row maximum
    const float got = dq::rounded_quotient(w, s, r, margin);
    const float want = std::rint(w / s);
    ++g_checked;
    const float t = w * r;
    const bool fast = std::fabs(t - std::rint(t)) < margin;
    g_fast += fast;
    g_rand += random;
    g_rand_fast += random && fast;
    if (!(got == want)) {
        if (g_bad < 10)
            std::printf("MISMATCH w=%a s=%a r=%a got %g want %g\n", w, s, r, got, want);
        ++g_bad;
    }
}

// every level and tie of one row scale, and random elements of the row
void check_scale(float amax, float s, float limit, int32_t jmax, std::mt19937_64& rng)
{
    const float r = 1.0f / s;
    const float margin = dq::quotient_margin(limit);
    const int32_t step = jmax > 2048 ? 7 : 1;  // wide codes: every 7th level, ends included
    for (int32_t j = -jmax - 1; j <= jmax; j += (j < -jmax + 2 || j > jmax - 3) ? 1 : step) {
        const float bases[2] = {((float)j + 0.5f) * s, (float)j * s};
        for (float base : bases) {
            float lo = base, hi = base;
            check(base, s, r, margin, amax);
            for (int k = 0; k < 6; ++k) {
                lo = std::nextafter(lo, -INFINITY);
                hi = std::nextafter(hi, INFINITY);
                check(lo, s, r, margin, amax);
                check(hi, s, r, margin, amax);
            }
        }
    }
    std::uniform_real_distribution<float> u(-1.0f, 1.0f);
    // (a reciprocal that overflows sends every element to the divide)
    for (int i = 0; i < 2000; ++i) check(u(rng) * amax, s, r, margin, amax, std::isfinite(r));
}

}  // namespace

int main()
{
    std::mt19937_64 rng(7);
    std::vector<float> maxima;
    for (int e = -149; e <= 127; e += 3) maxima.push_back(std::ldexp(1.37f, e));
    const float extra[] = {3.4028235e38f, 3.0e38f, 2.6e38f, 1.7e38f, 1.0e38f, 8.6e37f,
                           1.4e-45f, 2.8e-45f, 1.0e-40f, 1.17549435e-38f, 1.0f, 0.37f};
    for (float a : extra) maxima.push_back(a);
    uint64_t subnormal_r = 0, overflow_r = 0;
    for (int b = 2; b <= 15; ++b) {
        const int32_t qmax = (1 << (b - 1)) - 1, L = (1 << b) - 1;
        for (float a : maxima) {
            // symmetric scheme: s = fl32(max / qmax), |w / s| <= qmax + 1
            float s = a / (float)qmax;
            if (s > 0.0f && std::isfinite(s)) {
                const float r = 1.0f / s;
                subnormal_r += (r != 0.0f && std::fpclassify(r) == FP_SUBNORMAL);
                overflow_r += std::isinf(r);
                check_scale(a, s, (float)qmax + 1.0f, qmax, rng);
            }
            // asymmetric scheme: s = fl32(range / L), |w / s| <= L + 1
            s = a / (float)L;
            if (s > 0.0f && std::isfinite(s)) {
                const float r = 1.0f / s;
                subnormal_r += (r != 0.0f && std::fpclassify(r) == FP_SUBNORMAL);
                overflow_r += std::isinf(r);
                check_scale(a, s, (float)L + 1.0f, L, rng);
            }
        }
    }
    std::printf("checked %llu fast %llu bad %llu random %llu random_fast %llu subnormal_r %llu "
                "overflow_r %llu\n",
                (unsigned long long)g_checked, (unsigned long long)g_fast,
                (unsigned long long)g_bad, (unsigned long long)g_rand,
                (unsigned long long)g_rand_fast, (unsigned long long)subnormal_r,
                (unsigned long long)overflow_r);
    // both paths exercised (the divide near ties), the multiply taken for
    // nearly every random element, and the special reciprocals reached
    const bool ok = g_bad == 0 && g_fast > 0 && g_fast < g_checked &&
                    g_rand_fast * 100 > g_rand * 95 && subnormal_r > 0 && overflow_r > 0;
    return ok ? 0 : 1;
}
