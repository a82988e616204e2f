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

// The rotary step of the routing kernel (RouteRope), per round of items
// [j0, j0 + cnt) of a workgroup: all its threads turn the items' query rows
// into q_out and append each item's key (turned) and value row at pos, each
// rounded as by the standalone rotary kernel.  A rotary launch takes
// kRopeItemsPerWg items per workgroup (instead of one per 16-lane group), so
// the rows of a round are spread thin: a thread loads a batch of kRopeB pairs
// before it computes any (one batch for 4 items of G = 8 at d = 128), and the
// first batch is loaded before the workgroup computes the angles.
constexpr int kRopeB = 8;
constexpr int kRopeItemsPerWg = 4;

struct RopeRound {
    float x0[kRopeB], x1[kRopeB];
    float k0v, k1v, v0v, v1v;
};

// Loads of the batch starting at pair p0 (and, with the first, the key/value
// pairs: one per thread, kRopeItemsPerWg * d/2 <= NT).  Pairs index the rows
// j0*G .. (j0 + cnt)*G - 1 of q_new, d/2 = 2^hs pairs per row.
template <int NT>
__device__ inline void rope_round_load(const RouteRope& rr, int32_t j0, int32_t cnt, int32_t G,
                                       int32_t d, int hs, int32_t p0, bool first, RopeRound& L) {
    const int32_t half = d / 2, n = cnt * G * half;
#pragma unroll
    for (int r = 0; r < kRopeB; ++r) {  // pairs past n read pair 0 and go unused
        const int32_t e = p0 + static_cast<int32_t>(threadIdx.x) + r * NT < n
                              ? p0 + static_cast<int32_t>(threadIdx.x) + r * NT : 0;
        const int64_t row = static_cast<int64_t>(j0) * G + (e >> hs);
        const int32_t i = e & (half - 1);
        L.x0[r] = rr.q_new[row * d + i];
        L.x1[r] = rr.q_new[row * d + i + half];
    }
    if (!first) return;
    const int32_t e = static_cast<int32_t>(threadIdx.x) < cnt * half ? threadIdx.x : 0;
    const int64_t item = j0 + (e >> hs);
    const int32_t i = e & (half - 1);
    L.k0v = rr.k_new[item * d + i];
    L.k1v = rr.k_new[item * d + i + half];
    L.v0v = rr.v_new[item * d + i];
    L.v1v = rr.v_new[item * d + i + half];
}

// The round's rotary step, its first batch already in L; ends with the rows
// written and a barrier, so every wave's scores read them.
template <int NT>
__device__ inline void rope_round(const RouteRope& rr, const double* s_c, const double* s_s,
                                  int32_t j0, int32_t cnt, int32_t G, int32_t d, int32_t Hkv,
                                  int hs, RopeRound& L) {
    const int32_t half = d / 2, n = cnt * G * half;
    const int32_t dtype = rr.kv_f32 ? SR_KV_F32 : SR_KV_BF16;
    if (static_cast<int32_t>(threadIdx.x) < cnt * half) {
        const int32_t e = threadIdx.x, item = j0 + (e >> hs), i = e & (half - 1);
        const int32_t b = item / Hkv, g = item - b * Hkv;
        const int64_t at = b * rr.stride_b + g * rr.stride_h + rr.pos * rr.stride_t;
        double r0, r1;
        rope_turn(L.k0v, L.k1v, s_c[i], s_s[i], r0, r1);
        store_elem(rr.k_cache, at + i, r0, dtype);
        store_elem(rr.k_cache, at + i + half, r1, dtype);
        store_elem(rr.v_cache, at + i, L.v0v, dtype);
        store_elem(rr.v_cache, at + i + half, L.v1v, dtype);
    }
    for (int32_t p0 = 0;;) {
#pragma unroll
        for (int r = 0; r < kRopeB; ++r) {
            const int32_t e = p0 + static_cast<int32_t>(threadIdx.x) + r * NT;
            if (e >= n) break;
            const int64_t row = static_cast<int64_t>(j0) * G + (e >> hs);
            const int32_t i = e & (half - 1);
            double r0, r1;
            rope_turn(L.x0[r], L.x1[r], s_c[i], s_s[i], r0, r1);
            rr.q_out[row * d + i] = static_cast<float>(r0);
            rr.q_out[row * d + i + half] = static_cast<float>(r1);
        }
        p0 += NT * kRopeB;
        if (p0 >= n) break;
        rope_round_load<NT>(rr, j0, cnt, G, d, hs, p0, false, L);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the rows are written (in this XCD's L2)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // and no load of them moved above the stores
    __syncthreads();
}

// The decision step for a whole layer.  Item-major: each aligned 16-lane
// group scores every head of one item at a time (shared arithmetic in
// routing.h) and writes its flag; the workgroups stride over the items.
// Then one workgroup partitions the flags: the only workgroup of a
// one-workgroup launch (its flags stay in LDS), else the one that draws the
// last ticket (when `ticket` is given; a partition launch follows otherwise).
// The ticket starts at zero and is left at zero.  Without a work list the
// flags are the whole output (a decode launch that takes its decisions from
// them partitions the items itself).
template <int NT>
__global__ __launch_bounds__(NT) void k_route(
    const float* __restrict__ q, const float* __restrict__ k0, float tau,
    float* __restrict__ scores, uint8_t* __restrict__ flags, int32_t* __restrict__ work_list,
    int32_t* __restrict__ n_active, uint32_t* __restrict__ ticket, int32_t n_items, int32_t G,
    int32_t d, int32_t Hkv, RouteRope rr) {
    constexpr int GROUPS = NT / 16;
    static_assert(kRopeItemsPerWg * 64 <= NT, "one key/value pair per thread");
    const int hl = threadIdx.x & 15, hg = threadIdx.x >> 4;
    const bool rope = rr.q_new != nullptr;
    const int32_t ipw = rope ? kRopeItemsPerWg : GROUPS;  // items per workgroup and round
    // the rotary step's angles, once per workgroup
    __shared__ double s_c[64], s_s[64];  // d/2 <= 64
    // the rows scored: q, or the rotated rows this kernel writes (not restrict)
    const float* qs = q;
    const int hs = d == 128 ? 6 : 5;  // log2(d/2)
    RopeRound L;
    const int32_t j_first = static_cast<int32_t>(blockIdx.x) * ipw;
    auto count = [&](int32_t j0) { return n_items - j0 < ipw ? n_items - j0 : ipw; };
    if (rope) {
        // the first round's first batch is in flight while the angles are computed
        rope_round_load<NT>(rr, j_first, count(j_first), G, d, hs, 0, true, L);
        for (int i = threadIdx.x; i < d / 2; i += NT) rope_angle(rr.pos, rr.inv_freq, i, s_c[i], s_s[i]);
        __syncthreads();
        qs = rr.q_out;
    }
    if (gridDim.x == 1) {  // at most ipw items: flags through LDS, no device-wide publish
        __shared__ uint8_t s_flag[GROUPS];
        if (rope) rope_round<NT>(rr, s_c, s_s, 0, n_items, G, d, Hkv, hs, L);
        const bool own = hg < n_items;
        const int32_t j = own ? hg : n_items - 1;  // idle groups re-score the last item
        // (one round only: with the rotary step its rows are written by now)
        const bool sink = score_item16<8>(qs, k0, j, G, d, hl, tau, own ? scores : nullptr);
        if (own && hl == 0) {
            flags[j] = sink ? 1 : 0;
            s_flag[j] = sink ? 1 : 0;
        }
        if (work_list) partition_flags<NT>(s_flag, n_items, work_list, n_active);
        return;
    }
    const int32_t stride = static_cast<int32_t>(gridDim.x) * ipw;
    for (int32_t j0 = j_first; j0 < n_items; j0 += stride) {
        if (rope) {
            if (j0 != j_first) rope_round_load<NT>(rr, j0, count(j0), G, d, hs, 0, true, L);
            rope_round<NT>(rr, s_c, s_s, j0, count(j0), G, d, Hkv, hs, L);
        }
        const bool own = hg < ipw && j0 + hg < n_items;
        // idle groups re-score an item: without the rotary step the last; with
        // it the round's first, whose rotated rows are already written (an
        // earlier look at rows written in a later round could leave stale lines
        // in this CU's cache)
        const int32_t j = own ? j0 + hg : (rope ? j0 : n_items - 1);
        const bool sink = score_item16<8>(qs, k0, j, G, d, hl, tau, own ? scores : nullptr);
        if (own && hl == 0) {
            const uint8_t f = sink ? 1 : 0;
            // written through this XCD's L2, so the partitioning workgroup sees it
            __hip_atomic_store(flags + j, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's flag stores acknowledged
    if (!ticket) return;
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == gridDim.x - 1;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) *ticket = 0u;  // ready for the next call
    partition_flags<NT>(flags, n_items, work_list, n_active);
}

// The partition alone, after a many-workgroup k_route without a ticket.
template <int NT>
__global__ __launch_bounds__(NT) void k_partition(const uint8_t* __restrict__ flags,
                                                  int32_t* __restrict__ work_list,
                                                  int32_t* __restrict__ n_active,
                                                  int32_t n_items) {
    partition_flags<NT>(flags, n_items, work_list, n_active);
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

// One 256-thread workgroup per 16 groups (at most kRouteMaxWgs, which then
// stride).  Up to 16 groups that one workgroup also partitions; above, the
// workgroup that draws the last ticket does, or a second launch when there
// is no ticket.  Measured on MI355X under graph replay, this beats one
// 1024-thread workgroup over every item at every layer size from 32 query
// heads up (6.4 against 7.1 us at 512 heads, 8.8 against 246 us at 32768).
hipError_t launch_route(const sr_shape& s, const float* q, const float* k0, float tau,
                        float* scores, uint8_t* flags, int32_t* work_list, int32_t* n_active,
                        uint32_t* ticket, hipStream_t st, const RouteRope& rope) {
    constexpr int NT = 256, GROUPS = NT / 16;
    const int32_t n_items = s.batch * s.num_kv_heads;
    const int32_t G = s.num_q_heads / s.num_kv_heads;
    const int32_t ipw = rope.q_new ? kRopeItemsPerWg : GROUPS;  // as the kernel derives it
    const int32_t want = (n_items + ipw - 1) / ipw;
    const int32_t grid = want < kRouteMaxWgs ? want : kRouteMaxWgs;
    hipLaunchKernelGGL(k_route<NT>, dim3(grid), dim3(NT), 0, st, q, k0, tau, scores, flags,
                       work_list, n_active, ticket, n_items, G, s.head_dim, s.num_kv_heads, rope);
    // flags only (no list asked for: the decode partitions), or partitioned
    // already by the last workgroup or the only one
    if (!work_list || ticket || grid == 1) return hipGetLastError();
    // one tile of 4 flags per thread: 256 threads up to 1024 groups, 1024 above
    if (n_items <= 4 * 256)
        hipLaunchKernelGGL(k_partition<256>, dim3(1), dim3(256), 0, st, flags, work_list,
                           n_active, n_items);
    else
        hipLaunchKernelGGL(k_partition<1024>, dim3(1), dim3(1024), 0, st, flags, work_list,
                           n_active, n_items);
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
