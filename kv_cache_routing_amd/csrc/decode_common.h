// Device pieces shared by the two decode kernels (VALU and MFMA):
// the sink bypass, the work mapping, the workgroup -> split partial write and
// the last-arriver merge of split partials.
//
// Method: SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time
// steps: sink groups answer with the value at position 0 and read none of
// their cache; active groups run tiled attention with an online softmax, the
// context is split across workgroups and the splits are merged inside the
// kernel.  Eq. (1) of the paper (pith.science rendering of arXiv 2604.16883,
// Figure 1 caption) defines the result: the softmax-weighted sum of values.
#pragma once

#include "sr_internal.h"

namespace sr {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(m - M) as a merge weight; a state that saw no position (m = -inf)
// weighs nothing, even when M is -inf as well.
__device__ inline float merge_weight(float m, float M) {
    return m == kNegInf ? 0.f : fast_exp2(m - M);
}

template <int CTRL>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N in 4, 8, 16) with DPP; every lane of a
// group ends with the group's total.  All 64 lanes must be active.
template <int N>
__device__ inline float group_allreduce_sum(float x) {
    x += dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                          // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

template <int N>
__device__ inline float group_allreduce_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
    return x;
}

__device__ inline float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// What one workgroup owns: split `split` of the item at work-list slot `slot`.
struct WorkUnit {
    int32_t slot, split, splits, b, g;
    int64_t t0, t1;  // positions [t0, t1) of the item's cache
};

// Sink duty, then the work mapping.  Workgroup w first copies v0 into the G
// output rows of the sink at list position n_active + w (if there is one);
// then it takes split (w mod S) of active slot (w / S), S = splits per item.
// Returns false when the workgroup has no split to compute.
template <int D, int NT>
__device__ inline bool map_work(const DecodeArgs& a, WorkUnit& u) {
    const int32_t n_items = a.batch * a.num_kv_heads;
    const int32_t n_act = a.routed ? *a.n_active : n_items;
    const int32_t wg = blockIdx.x;
    const int32_t G = a.group;
    if (a.routed) {
        const int32_t ss = n_act + wg;
        if (ss < n_items) {
            const int32_t j = a.work_list[ss];
            const int32_t b = j / a.num_kv_heads, g = j - b * a.num_kv_heads;
            const float* src = a.v0 + static_cast<int64_t>(j) * D;
            float* dst = a.out + (static_cast<int64_t>(b) * a.num_q_heads +
                                  static_cast<int64_t>(g) * G) * D;
            for (int x = threadIdx.x; x < G * D; x += NT) dst[x] = src[x % D];
        }
    }
    if (n_act <= 0) return false;
    const int32_t S = splits_for(a.fixed_splits, a.grid, a.split_cap, n_act);
    const int32_t slot = wg / S;
    if (slot >= n_act) return false;
    u.slot = slot;
    u.split = wg - slot * S;
    u.splits = S;
    const int32_t item = a.routed ? a.work_list[slot] : slot;
    u.b = item / a.num_kv_heads;
    u.g = item - u.b * a.num_kv_heads;
    const int64_t L = split_len(a.seq_len, S);
    u.t0 = static_cast<int64_t>(u.split) * L;
    const int64_t e = u.t0 + L;
    u.t1 = e < a.seq_len ? e : a.seq_len;
    if (u.t0 > u.t1) u.t0 = u.t1;  // empty split
    return true;
}

// Merge the per-wave states held in LDS (s_m/s_l [NW][GP], s_acc [NW][GP][D])
// into this workgroup's split partial.  With one split per item the partial
// is final and goes straight to `out`; otherwise it is stored, published with
// an agent-scope release, and the last workgroup of the item to take a ticket
// merges all S partials in ascending split order and writes `out`.
template <int D, int GP, int NW>
__device__ inline void finish_split(const DecodeArgs& a, const WorkUnit& u,
                                    const float (*s_m)[GP], const float (*s_l)[GP],
                                    const float (*s_acc)[GP][D]) {
    constexpr int NT = NW * 64;
    const int32_t G = a.group;
    float* out_item = a.out + (static_cast<int64_t>(u.b) * a.num_q_heads +
                               static_cast<int64_t>(u.g) * G) * D;
    const int64_t wg = blockIdx.x;

    if (u.splits == 1) {
        for (int x = threadIdx.x; x < G * D; x += NT) {
            const int h = x / D, i = x - (x / D) * D;
            float M = kNegInf;
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
            float A = 0.f, L = 0.f;
            for (int w = 0; w < NW; ++w) {
                const float wt = merge_weight(s_m[w][h], M);
                A += wt * s_acc[w][h][i];
                L += wt * s_l[w][h];
            }
            out_item[x] = A / L;
        }
        return;
    }

    float* pml = a.part_ml + wg * 2 * GP;
    float* pacc = a.part_acc + wg * GP * D;
    for (int x = threadIdx.x; x < GP * D; x += NT) {
        const int h = x / D, i = x - (x / D) * D;
        float M = kNegInf;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
        float A = 0.f, L = 0.f;
        for (int w = 0; w < NW; ++w) {
            const float wt = merge_weight(s_m[w][h], M);
            A += wt * s_acc[w][h][i];
            L += wt * s_l[w][h];
        }
        pacc[x] = A;
        if (i == 0) {
            pml[h] = M;
            pml[GP + h] = L;
        }
    }

    __shared__ int s_last;
    __threadfence();  // release this workgroup's partial at agent scope
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(a.tickets + u.slot, 1u);
        s_last = prev == static_cast<uint32_t>(u.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire the other workgroups' partials

    constexpr int CH = 64;
    __shared__ float s_M[GP], s_L[GP];
    __shared__ float s_w[CH][GP];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t S = u.splits;
    const float* ml0 = a.part_ml + static_cast<int64_t>(u.slot) * S * 2 * GP;
    const float* acc0 = a.part_acc + static_cast<int64_t>(u.slot) * S * GP * D;

    for (int h = wave; h < GP; h += NW) {
        float M = kNegInf;
        for (int s = lane; s < S; s += 64) M = fmaxf(M, ml0[static_cast<int64_t>(s) * 2 * GP + h]);
        M = wave_max(M);
        if (lane == 0) s_M[h] = M;
    }
    constexpr int PER = (GP * D + NT - 1) / NT;
    float A[PER];
    for (int k = 0; k < PER; ++k) A[k] = 0.f;
    float Lh = 0.f;
    __syncthreads();
    for (int c0 = 0; c0 < S; c0 += CH) {
        const int n = S - c0 < CH ? S - c0 : CH;
        for (int x = threadIdx.x; x < CH * GP; x += NT) {
            const int k = x / GP, h = x - (x / GP) * GP;
            s_w[k][h] = k < n ? merge_weight(ml0[static_cast<int64_t>(c0 + k) * 2 * GP + h], s_M[h])
                              : 0.f;
        }
        __syncthreads();
        for (int k = 0; k < PER; ++k) {
            const int x = threadIdx.x + k * NT;
            if (x < GP * D) {
                const int h = x / D;
                const float* p = acc0 + static_cast<int64_t>(c0) * GP * D + x;
                float acc = A[k];
                for (int s = 0; s < n; ++s) acc += s_w[s][h] * p[static_cast<int64_t>(s) * GP * D];
                A[k] = acc;
            }
        }
        if (threadIdx.x < GP) {
            const int h = threadIdx.x;
            const float* p = ml0 + static_cast<int64_t>(c0) * 2 * GP + GP + h;
            for (int s = 0; s < n; ++s) Lh += s_w[s][h] * p[static_cast<int64_t>(s) * 2 * GP];
        }
        __syncthreads();
    }
    if (threadIdx.x < GP) s_L[threadIdx.x] = Lh;
    __syncthreads();
    for (int k = 0; k < PER; ++k) {
        const int x = threadIdx.x + k * NT;
        if (x < G * D) out_item[x] = A[k] / s_L[x / D];
    }
    if (threadIdx.x == 0) a.tickets[u.slot] = 0u;  // ready for the next call
}

}  // namespace sr
