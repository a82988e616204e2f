// Prefill-side sink record and decode-side routing for libsinkroute.
//
// SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time steps:
// the key at position 0 is kept from prefill; at decode the rotated query is
// compared with it and each GQA KV group is sent either down the sink bypass
// or down the attention path before any of its cache is read.  The score is
// a cosine (README routing controls; pith.science rendering of arXiv
// 2604.16883, Figure 10: cos(q, K_BOS) judged per KV group).
#include "decode_common.h"

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

template <typename X>
__device__ inline X wave_sum(X x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxItems = 32768;
constexpr int kHeadsPerPass = kRouteThreads / 16;  // one 16-lane group per head
constexpr int kPassUnroll = 4;                       // heads per group per round

// One workgroup.  Phase 1: a 16-lane group per query head loads its query row
// and its group's k0 row (d/16 contiguous floats per lane, all loads of a
// round in flight together), reduces <q,k0>, |q|^2, |k0|^2 with DPP and
// writes the cosine; a head below tau marks its item active in LDS.
// Phase 2: mask, then a stable partition of the items (active first) by
// ballot prefix counts.
__global__ __launch_bounds__(kRouteThreads) void k_route(
    const float* __restrict__ q, const float* __restrict__ k0, float tau,
    float* __restrict__ scores, uint8_t* __restrict__ mask, int32_t* __restrict__ work_list,
    int32_t* __restrict__ n_active, int32_t B, int32_t Hq, int32_t Hkv, int32_t d) {
    __shared__ uint8_t s_sink[kMaxItems];
    __shared__ int32_t s_wave_a[kRouteWaves], s_wave_s[kRouteWaves];
    __shared__ int32_t s_count;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t G = Hq / Hkv;
    const int32_t n_items = B * Hkv;
    const int64_t n_heads = static_cast<int64_t>(n_items) * G;  // head j*G + i belongs to item j
    const int hl = tid & 15, hg = tid >> 4;

    for (int32_t j = tid; j < n_items; j += kRouteThreads) s_sink[j] = 1;
    if (tid == 0) s_count = 0;
    __syncthreads();

    for (int64_t base = 0; base < n_heads; base += kHeadsPerPass * kPassUnroll) {
        float qk[kPassUnroll], qq[kPassUnroll], kk[kPassUnroll];
#pragma unroll
        for (int r = 0; r < kPassUnroll; ++r) {
            qk[r] = qq[r] = kk[r] = 0.f;
            const int64_t hh = base + hg + static_cast<int64_t>(r) * kHeadsPerPass;
            if (hh < n_heads) {
                const float* qp = q + hh * d;
                const float* kp = k0 + (hh / G) * d;
                for (int e = 4 * hl; e < d; e += 64) {
                    const float4 x = *reinterpret_cast<const float4*>(qp + e);
                    const float4 y = *reinterpret_cast<const float4*>(kp + e);
                    qk[r] += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
                    qq[r] += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
                    kk[r] += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kPassUnroll; ++r) {
            const float dot = group_allreduce_sum<16>(qk[r]);
            const float nq = group_allreduce_sum<16>(qq[r]);
            const float nk = group_allreduce_sum<16>(kk[r]);
            const int64_t hh = base + hg + static_cast<int64_t>(r) * kHeadsPerPass;
            if (hh < n_heads && hl == 0) {
                const float den = sqrtf(nq) * sqrtf(nk);
                const float c = den > 0.f ? dot / den : 0.f;
                scores[hh] = c;
                if (!(c >= tau)) s_sink[hh / G] = 0;  // one dissenting head keeps the group active
            }
        }
    }
    __syncthreads();

    int32_t local = 0;
    for (int32_t j = tid; j < n_items; j += kRouteThreads) {
        mask[j] = s_sink[j];
        local += s_sink[j] ? 0 : 1;
    }
    local = wave_sum(local);
    if (lane == 0) atomicAdd(&s_count, local);
    __syncthreads();
    const int32_t n_act = s_count;

    // stable partition: active items keep their order, then sinks keep theirs
    int32_t base_a = 0, base_s = n_act;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int32_t c0 = 0; c0 < n_items; c0 += kRouteThreads) {
        const int32_t j = c0 + tid;
        const bool in = j < n_items;
        const bool is_a = in && !s_sink[j];
        const bool is_s = in && s_sink[j];
        const uint64_t ba = __ballot(is_a), bs = __ballot(is_s);
        if (lane == 0) {
            s_wave_a[wave] = __popcll(ba);
            s_wave_s[wave] = __popcll(bs);
        }
        __syncthreads();
        int32_t pa = base_a, ps = base_s, ta = 0, ts = 0;
        for (int w = 0; w < kRouteWaves; ++w) {
            if (w < wave) {
                pa += s_wave_a[w];
                ps += s_wave_s[w];
            }
            ta += s_wave_a[w];
            ts += s_wave_s[w];
        }
        if (is_a) work_list[pa + __popcll(ba & lt)] = j;
        if (is_s) work_list[ps + __popcll(bs & lt)] = j;
        base_a += ta;
        base_s += ts;
        __syncthreads();
    }
    if (tid == 0) n_active[0] = n_act;
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
