// Packed row geometry, shared by the host-only sources (file format) and the
// kernel launchers; no HIP dependency.  A packed row holds ceil(K * bits / 8)
// bytes of codes, padded with zero bits to a multiple of 128 bytes.
#pragma once

#include <stdint.h>

namespace dq {

inline int64_t packed_row_words(int64_t K, int bits)
{
    return ((K * bits + 7) / 8 + 127) / 128 * 128 / 4;
}

}  // namespace dq
