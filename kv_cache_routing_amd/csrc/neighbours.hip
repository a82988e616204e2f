// Decode-step neighbours of the routed attention: rotary embedding of the new
// token's query and key, and the append of its key and value to the caches.
//
// SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time steps:
// the routing score compares the RoPE-rotated query with the key kept at
// position 0, so every decode step first rotates the new query and key and
// appends the new key/value; position 0 itself is never rotated (angle 0).
// Rotary form (not printed on the pages; Hugging Face Llama convention):
// element i is paired with element i + d/2 and both turn by pos * inv_freq[i].
#include "rope.h"

namespace sr {
namespace {

// One thread per pair (i, i + d/2) of every query row, key row and value row.
__global__ void k_rope_append(const float* __restrict__ q_new, const float* __restrict__ k_new,
                              const float* __restrict__ v_new, const float* __restrict__ inv_freq,
                              int64_t pos, float* __restrict__ q_out, void* k_cache, void* v_cache,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t sb, int64_t sh,
                              int64_t st, int32_t dtype) {
    const int32_t half = d / 2;
    const int64_t nq = static_cast<int64_t>(B) * Hq * half;
    const int64_t nk = static_cast<int64_t>(B) * Hkv * half;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= nq + 2 * nk) return;
    int64_t row, kind;  // kind 0: query, 1: key, 2: value
    if (e < nq) {
        kind = 0;
        row = e / half;
    } else if (e < nq + nk) {
        kind = 1;
        row = (e - nq) / half;
    } else {
        kind = 2;
        row = (e - nq - nk) / half;
    }
    const int32_t i = static_cast<int32_t>(e % half);
    const float* src = kind == 0 ? q_new : (kind == 1 ? k_new : v_new);
    const double x0 = src[row * d + i], x1 = src[row * d + i + half];
    double r0 = x0, r1 = x1;
    if (kind != 2) {
        double c, s;
        rope_angle(pos, inv_freq, i, c, s);
        rope_turn(x0, x1, c, s, r0, r1);
    }
    if (kind == 0) {
        q_out[row * d + i] = static_cast<float>(r0);
        q_out[row * d + i + half] = static_cast<float>(r1);
        return;
    }
    const int64_t b = row / Hkv, g = row - b * Hkv;
    const int64_t at = b * sb + g * sh + pos * st;
    void* cache = kind == 1 ? k_cache : v_cache;
    store_elem(cache, at + i, r0, dtype);
    store_elem(cache, at + i + half, r1, dtype);
}

}  // namespace

hipError_t launch_rope_append(const sr_shape& s, const float* q_new, const float* k_new,
                              const float* v_new, const float* inv_freq, int64_t pos,
                              float* q_out, void* k_cache, void* v_cache, hipStream_t st) {
    const int64_t n = static_cast<int64_t>(s.batch) * (s.num_q_heads + 2 * s.num_kv_heads) *
                      (s.head_dim / 2);
    const int threads = 256;
    const unsigned blocks = static_cast<unsigned>((n + threads - 1) / threads);
    hipLaunchKernelGGL(k_rope_append, dim3(blocks), dim3(threads), 0, st, q_new, k_new, v_new,
                       inv_freq, pos, q_out, k_cache, v_cache, s.batch, s.num_q_heads,
                       s.num_kv_heads, s.head_dim, s.stride_b, s.stride_h, s.stride_t,
                       s.kv_dtype);
    return hipGetLastError();
}

}  // namespace sr
