// Rotary embedding and cache-row stores shared by the standalone rotary +
// append kernel and the decode launch that fuses them, so both forms produce
// the same bits.
//
// SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time steps:
// the routing score compares the RoPE-rotated query with the key kept at
// position 0.  Rotary form (not printed on the pages; Hugging Face Llama
// convention): element i is paired with element i + d/2 and both turn by the
// angle pos * inv_freq[i].  Angles, sines, cosines and the rotation run in
// fp64; each result is rounded once, to fp32 for the query and to the cache
// dtype for the key.
#pragma once

#include "angle.h"
#include "sr_internal.h"

namespace sr {

// fp64 -> bf16 with one rounding to nearest even: truncate to fp32 and keep a
// sticky bit (round to odd, 24 >= 8 + 2 bits), then round the fp32 bits.
__device__ inline uint16_t bf16_from_double(double x) {
    const float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if (static_cast<double>(f) != x) u |= 1u;
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline void store_elem(void* base, int64_t idx, double x, int32_t dtype) {
    if (dtype == SR_KV_F32)
        static_cast<float*>(base)[idx] = static_cast<float>(x);
    else
        static_cast<uint16_t*>(base)[idx] = bf16_from_double(x);
}

// cos and sin of the angle pos * inv_freq[i] (the product rounded once in fp64).
__device__ inline void rope_angle(int64_t pos, const float* inv_freq, int32_t i, double& c,
                                  double& s) {
    angle_sincos(static_cast<double>(pos) * static_cast<double>(inv_freq[i]), s, c);
}

// The pair (x0, x1) turned by the angle with cosine c and sine s; the fused
// multiply-adds are explicit so that every caller rounds alike.
__device__ inline void rope_turn(double x0, double x1, double c, double s, double& r0,
                                 double& r1) {
    r0 = fma(x0, c, -(x1 * s));
    r1 = fma(x1, c, x0 * s);
}

}  // namespace sr
