// Prefill-side sink record and decode-side routing for libsinkroute.
//
// SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time steps:
// the key at position 0 is kept from prefill; at decode the rotated query is
// compared with it and each GQA KV group is sent either down the sink bypass
// or down the attention path before any of its cache is read.  The score is
// a cosine (README routing controls; pith.science rendering of arXiv
// 2604.16883, Figure 10: cos(q, K_BOS) judged per KV group).
#include "routing.h"

namespace sr {
namespace {

__device__ inline float load_elem(const void* base, int64_t idx, int32_t dtype) {
    if (dtype == SR_KV_F32) return static_cast<const float*>(base)[idx];
    uint32_t bits = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float(bits << 16);
}

// k0[j][i] = K[b][g][0][i], v0[j][i] = V[b][g][0][i] (exact widening to fp32).
__global__ void k_record(const void* k, const void* v, float* k0, float* v0, int32_t Hkv,
                         int32_t d, int64_t sb, int64_t sh, int32_t dtype, int64_t n) {
    int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= n) return;
    int64_t j = e / d;
    int32_t i = static_cast<int32_t>(e - j * d);
    int64_t b = j / Hkv, g = j - b * Hkv;
    int64_t src = b * sb + g * sh + i;  // position 0
    k0[e] = load_elem(k, src, dtype);
    v0[e] = load_elem(v, src, dtype);
}

constexpr int kRouteThreads = 1024;
constexpr int kMaxItems = 32768;

// One workgroup: every head's cosine and every group's decision (shared
// arithmetic in routing.h), then the stable active-first partition.
__global__ __launch_bounds__(kRouteThreads) void k_route(
    const float* __restrict__ q, const float* __restrict__ k0, float tau,
    float* __restrict__ scores, uint8_t* __restrict__ mask, int32_t* __restrict__ work_list,
    int32_t* __restrict__ n_active, int32_t B, int32_t Hq, int32_t Hkv, int32_t d) {
    __shared__ uint8_t s_sink[kMaxItems];
    __shared__ int32_t s_wa[kRouteThreads / 64], s_ws[kRouteThreads / 64];
    const int32_t G = Hq / Hkv;
    const int32_t n_items = B * Hkv;
    route_items<kRouteThreads, 4>(q, k0, tau, n_items, G, d, s_sink, scores, mask);
    if (n_items <= kRouteThreads) {
        int32_t pos;
        const int32_t n_act = partition_one_pass<kRouteThreads>(s_sink, n_items, s_wa, s_ws, pos);
        if (static_cast<int32_t>(threadIdx.x) < n_items) work_list[pos] = threadIdx.x;
        if (threadIdx.x == 0) n_active[0] = n_act;
        return;
    }
    const int32_t n_act = count_active<kRouteThreads>(s_sink, n_items, s_wa);
    partition_items<kRouteThreads>(s_sink, n_items, n_act, s_wa, s_ws,
                                   [&](int32_t pos, int32_t j) { work_list[pos] = j; });
    if (threadIdx.x == 0) n_active[0] = n_act;
}

__global__ void k_zero(uint32_t* p, int64_t n) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_record(const sr_shape& s, const void* k, const void* v, float* k0, float* v0,
                         hipStream_t st) {
    const int64_t n = static_cast<int64_t>(s.batch) * s.num_kv_heads * s.head_dim;
    const int threads = 256;
    const unsigned blocks = static_cast<unsigned>((n + threads - 1) / threads);
    hipLaunchKernelGGL(k_record, dim3(blocks), dim3(threads), 0, st, k, v, k0, v0,
                       s.num_kv_heads, s.head_dim, s.stride_b, s.stride_h, s.kv_dtype, n);
    return hipGetLastError();
}

hipError_t launch_route(const sr_shape& s, const float* q, const float* k0, float tau,
                        float* scores, uint8_t* mask, int32_t* work_list, int32_t* n_active,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_route, dim3(1), dim3(kRouteThreads), 0, st, q, k0, tau, scores, mask,
                       work_list, n_active, s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim);
    return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
    const int64_t n = static_cast<int64_t>(bytes / 4);
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const unsigned blocks = static_cast<unsigned>((n + threads - 1) / threads);
    hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(threads), 0, st, static_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

}  // namespace sr
