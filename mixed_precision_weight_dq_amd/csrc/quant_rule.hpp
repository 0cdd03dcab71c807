// The quantizer's rounded quotient rint(fl32(w / s)) (round half to even, as
// numpy's round in the "量化" tutorial's Step 1 code), without an IEEE divide
// per element where that provably gives the same integer.
//
// r = fl32(1 / s) (one IEEE divide per row) has a relative error of at most
// 2^-24 when 1/s is a normal number; when it is subnormal (s > 2^126), 1/s is
// still above 2^-128 (s is finite), so its absolute error of at most 2^-150 is
// a relative error below 2^-22.  Then t' = fl32(w * r) lies within
// (2^-22 + 2^-24 + 2^-46) |w / s| of w / s, and fl32(w / s) within
// 2^-24 |w / s|, so |t' - fl32(w / s)| < 1.5 * 2^-22 |w / s| <= 1.5 * 2^-22 * limit,
// where limit bounds |w / s| over the row (qmax + 1 in the symmetric scheme,
// L + 1 in the asymmetric one).  So rint(t') = rint(fl32(w / s)) unless a
// half-integer lies within 2^-21 * limit of t': the margin below.  Those
// elements (and any non-finite t', as when 1/s overflows for a tiny s) take
// the IEEE divide.
//
// Plain host/device code: the kernels inline it, and a host test runs it over
// every tie neighbourhood against the IEEE divide.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

namespace dq {

// Distance from the nearest half-integer below which t' is not trusted.
__host__ __device__ __forceinline__ float quotient_margin(float limit)
{
    return 0.5f - ldexpf(limit, -21);
}

// rint(fl32(w / s)) given r = fl32(1 / s) and margin = quotient_margin(limit).
__host__ __device__ __forceinline__ float rounded_quotient(float w, float s, float r, float margin)
{
    const float t = w * r;
    float q = rintf(t);
    if (!(fabsf(t - q) < margin)) q = rintf(w / s);  // near a tie, or not finite
    return q;
}

}  // namespace dq
