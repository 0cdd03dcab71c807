// A plain streaming read: not a step of the method, the yardstick for the
// bandwidth-bound kernels of this library.  It moves the bytes a decode GEMV
// moves and does nothing else, so its rate at a given size is what a kernel
// bound by HBM can reach there (launch, latency and ramp included).
//
// Workgroup p reads the 16-byte pieces [n16 p / nparts, n16 (p + 1) / nparts)
// with four loads in flight per thread and writes the XOR of their 32-bit
// words to partial[p] (XOR is order independent, so the result is exact and
// a test can check every byte was read).
#include "common.hpp"
#include "launch.hpp"

namespace dq {

namespace {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const uint4* __restrict__ buf, int64_t n16, int64_t nparts, uint32_t* __restrict__ partial)
{
    const int64_t p = blockIdx.x;
    const int64_t begin = n16 * p / nparts, end = n16 * (p + 1) / nparts;
    constexpr int64_t T = kStreamThreads;
    uint32_t acc = 0;
    int64_t i = begin + threadIdx.x;
    for (; i + 3 * T < end; i += 4 * T) {
        const uint4 a = buf[i], b = buf[i + T], c = buf[i + 2 * T], d = buf[i + 3 * T];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
               (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < end; i += T) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t wx[kStreamThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) wx[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kStreamThreads / kWave; ++w) r ^= wx[w];
        partial[p] = r;
    }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int64_t nparts,
                              hipStream_t stream)
{
    stream_read_kernel<<<dim3((unsigned)nparts), dim3(kStreamThreads), 0, stream>>>(
        static_cast<const uint4*>(buf), bytes / 16, nparts, partial);
    return hipGetLastError();
}

}  // namespace dq
