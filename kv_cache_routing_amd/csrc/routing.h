// Routing arithmetic shared by the routing kernel and the fused route+decode
// prologue, so both take bit-identical decisions.
//
// SinkRouter README (github.com/streamer-AP/SinkRouter): at decode each GQA KV
// group is scored by the cosine between the rotated query and the key kept at
// position 0 (routing-controls section: a cosine threshold), and is sent down
// the sink bypass or the attention path before its cache is read
// (decode-time steps); pith.science rendering of arXiv 2604.16883, Figure 10:
// cos(q, K_BOS) judged at the KV-group level.  Reading: a group is a sink only
// when every one of its heads has cos >= tau; a zero norm scores 0.
#pragma once

#include "decode_common.h"

namespace sr {

// Cosines of U query heads, one head per aligned 16-lane group: head
// first + r * stride (r < U) in group lane hl.  Lane hl accumulates elements
// 4*hl + 64*k with explicit fmaf in a fixed order, then a fixed DPP tree
// reduces the group, so a head's score does not depend on which kernel or
// which lane group computed it.  Every load is issued before the first
// product and none sits under a branch (a head past the end re-reads the
// last head, whose score the caller ignores; for d = 64 the second half
// re-reads the first and is not summed), so one wait covers them all.
// Slots r >= n_live (no lane group has a head there; uniform across the
// workgroup) skip the arithmetic and leave c[r] undefined.
// d is 64 or 128.  All 64 lanes of the wave must be active.
template <int U>
__device__ inline void head_cosines16(const float* __restrict__ q, const float* __restrict__ k0,
                                      int32_t first, int32_t stride, int32_t n_heads, int32_t G,
                                      int32_t d, int hl, int32_t n_live, float (&c)[U]) {
    float4 xq[U][2], xk[U][2];
#pragma unroll
    for (int r = 0; r < U; ++r) {
        int32_t hh = first + r * stride;
        hh = hh < n_heads ? hh : n_heads - 1;
        const float* qp = q + static_cast<int64_t>(hh) * d;
        const float* kp = k0 + static_cast<int64_t>(hh / G) * d;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 4 * hl + (64 * k < d ? 64 * k : 0);
            xq[r][k] = *reinterpret_cast<const float4*>(qp + e);
            xk[r][k] = *reinterpret_cast<const float4*>(kp + e);
        }
    }
#pragma unroll
    for (int r = 0; r < U; ++r) {
        c[r] = 0.f;
        if (r >= n_live) continue;
        float qk = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (64 * k < d) {
                const float4 x = xq[r][k], y = xk[r][k];
                qk = fmaf(x.x, y.x, qk);
                qk = fmaf(x.y, y.y, qk);
                qk = fmaf(x.z, y.z, qk);
                qk = fmaf(x.w, y.w, qk);
                qq = fmaf(x.x, x.x, qq);
                qq = fmaf(x.y, x.y, qq);
                qq = fmaf(x.z, x.z, qq);
                qq = fmaf(x.w, x.w, qq);
                kk = fmaf(y.x, y.x, kk);
                kk = fmaf(y.y, y.y, kk);
                kk = fmaf(y.z, y.z, kk);
                kk = fmaf(y.w, y.w, kk);
            }
        }
        const float dot = group_allreduce_sum<16>(qk);
        const float nq = group_allreduce_sum<16>(qq);
        const float nk = group_allreduce_sum<16>(kk);
        const float den = sqrtf(nq) * sqrtf(nk);
        c[r] = den > 0.f ? dot / den : 0.f;
    }
}

// Every head of item j (G heads, rows j*G .. j*G + G - 1 of q) against the
// item's position-0 key, by one aligned 16-lane group; returns, in every lane,
// whether every head has cos >= tau.  The products, their order and the
// reduction tree are head_cosines16's, so each score is the one that function
// gives bit for bit; the key row is loaded and its norm reduced once for all
// G heads.  Heads go U at a time with every load of a batch issued before its
// arithmetic; the slots of a short last batch re-read the batch's first head
// and are not computed (the batch size is the same in every lane).  Lane r of
// the group writes the batch's r-th score when scores is non-null.  d is 64
// or 128.  All 64 lanes of the wave must be active.
template <int U>
__device__ inline bool score_item16(const float* __restrict__ q, const float* __restrict__ k0,
                                    int32_t j, int32_t G, int32_t d, int hl, float tau,
                                    float* scores) {
    const float* kp = k0 + static_cast<int64_t>(j) * d;
    float4 xk[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) xk[k] = *reinterpret_cast<const float4*>(kp + 4 * hl + (64 * k < d ? 64 * k : 0));
    float kk = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (64 * k < d) {
            const float4 y = xk[k];
            kk = fmaf(y.x, y.x, kk);
            kk = fmaf(y.y, y.y, kk);
            kk = fmaf(y.z, y.z, kk);
            kk = fmaf(y.w, y.w, kk);
        }
    }
    const float sk = sqrtf(group_allreduce_sum<16>(kk));
    bool sink = true;
    for (int32_t c0 = 0; c0 < G; c0 += U) {
        const int32_t n_h = G - c0 < U ? G - c0 : U;
        const float* qb = q + (static_cast<int64_t>(j) * G + c0) * d;
        float4 xq[U][2];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const float* qp = qb + static_cast<int64_t>(r < n_h ? r : 0) * d;
#pragma unroll
            for (int k = 0; k < 2; ++k)
                xq[r][k] = *reinterpret_cast<const float4*>(qp + 4 * hl + (64 * k < d ? 64 * k : 0));
        }
        float mine = 0.f;
#pragma unroll
        for (int r = 0; r < U; ++r) {
            if (r >= n_h) break;
            float qk = 0.f, qq = 0.f;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (64 * k < d) {
                    const float4 x = xq[r][k], y = xk[k];
                    qk = fmaf(x.x, y.x, qk);
                    qk = fmaf(x.y, y.y, qk);
                    qk = fmaf(x.z, y.z, qk);
                    qk = fmaf(x.w, y.w, qk);
                    qq = fmaf(x.x, x.x, qq);
                    qq = fmaf(x.y, x.y, qq);
                    qq = fmaf(x.z, x.z, qq);
                    qq = fmaf(x.w, x.w, qq);
                }
            }
            const float dot = group_allreduce_sum<16>(qk);
            const float nq = group_allreduce_sum<16>(qq);
            const float den = sqrtf(nq) * sk;
            const float c = den > 0.f ? dot / den : 0.f;
            sink = sink && c >= tau;
            if (hl == r) mine = c;
        }
        if (scores && hl < n_h) scores[static_cast<int64_t>(j) * G + c0 + hl] = mine;
    }
    return sink;
}

// Stable partition of the items from their flags (1 = sink) in global
// memory, by one workgroup of NT threads: active items in ascending order at
// list positions [0, n_act), sinks in ascending order after them; *n_active =
// n_act.  Thread t takes items 4t .. 4t + 3 of each tile of 4*NT and one
// block-wide scan of packed (sink << 16 | active) counts places them; layers
// of more than one tile count the active items in a first pass.  Starts and
// ends with a workgroup barrier.
template <int NT>
__device__ inline void partition_flags(const uint8_t* flags, int32_t n_items, int32_t* list,
                                       int32_t* n_active) {
    constexpr int NWV = NT / 64, TILE = 4 * NT;
    static_assert(TILE < 65536, "packed 16-bit counts");
    __shared__ int32_t s_tot[NWV];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    int32_t n_act = 0;
    if (n_items > TILE) {
        int32_t local = 0;
        for (int32_t j = threadIdx.x; j < n_items; j += NT) local += flags[j] ? 0 : 1;
        for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
        if (lane == 0) s_tot[wave] = local;
        __syncthreads();
        for (int w = 0; w < NWV; ++w) n_act += s_tot[w];
        __syncthreads();
    }
    int32_t base_a = 0, base_s = 0;
    for (int32_t t0 = 0; t0 < n_items; t0 += TILE) {
        const int32_t j0 = t0 + 4 * static_cast<int32_t>(threadIdx.x);
        uint32_t f = 0;  // bit e: item j0 + e is a sink; bit 4 + e: it exists
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j0 + e < n_items) f |= (flags[j0 + e] ? 1u : 0u) << e | 1u << (4 + e);
        const int32_t cs = __popc(f & 0xFu), ca = __popc(f >> 4) - cs;
        const int32_t mine = cs << 16 | ca;
        int32_t x = mine;  // inclusive scan over the wave
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_tot[wave] = x;
        __syncthreads();
        int32_t before = 0, tile = 0;
        for (int w = 0; w < NWV; ++w) {
            if (w < wave) before += s_tot[w];
            tile += s_tot[w];
        }
        __syncthreads();
        const int32_t ex = x - mine + before;
        if (n_items <= TILE) n_act = tile & 0xFFFF;  // one tile: its total is the count
        int32_t pa = base_a + (ex & 0xFFFF), ps = n_act + base_s + (ex >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (!(f >> (4 + e) & 1u)) break;
            if (f >> e & 1u) list[ps++] = j0 + e;
            else list[pa++] = j0 + e;
        }
        base_a += tile & 0xFFFF;
        base_s += tile >> 16;
    }
    if (threadIdx.x == 0) *n_active = n_act;
}

// Scores of every head of the layer (B*Hq heads of G per item), computed by
// NT threads; s_sink[j] ends 1 iff every head of item j has cos >= tau.
// Heads and items are written to `scores` / `mask` when those are non-null.
// Ends with a workgroup barrier.
template <int NT, int U>
__device__ inline void route_items(const float* __restrict__ q, const float* __restrict__ k0,
                                   float tau, int32_t n_items, int32_t G, int32_t d,
                                   uint8_t* s_sink, float* scores, uint8_t* mask) {
    constexpr int GROUPS = NT / 16;
    const int tid = threadIdx.x, hl = tid & 15, hg = tid >> 4;
    const int32_t n_heads = n_items * G;
    for (int32_t j = tid; j < n_items; j += NT) s_sink[j] = 1;
    __syncthreads();
    for (int32_t base = 0; base < n_heads; base += GROUPS * U) {
        float c[U];
        const int32_t n_live = (n_heads - base + GROUPS - 1) / GROUPS;  // same for every thread
        head_cosines16<U>(q, k0, base + hg, GROUPS, n_heads, G, d, hl, n_live, c);
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int32_t hh = base + hg + r * GROUPS;
            if (hh < n_heads && hl == 0) {
                if (scores) scores[hh] = c[r];
                if (!(c[r] >= tau)) s_sink[hh / G] = 0;  // one dissenting head keeps it active
            }
        }
    }
    __syncthreads();
    if (mask)
        for (int32_t j = tid; j < n_items; j += NT) mask[j] = s_sink[j];
}

// Number of active items (s_sink[j] == 0), from every thread.
template <int NT>
__device__ inline int32_t count_active(const uint8_t* s_sink, int32_t n_items, int32_t* s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t local = 0;
    for (int32_t j = threadIdx.x; j < n_items; j += NT) local += s_sink[j] ? 0 : 1;
    for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
    if (lane == 0) s_tmp[wave] = local;
    __syncthreads();
    int32_t n = 0;
    for (int w = 0; w < NT / 64; ++w) n += s_tmp[w];
    __syncthreads();
    return n;
}

// Count and stable partition in one pass when every item has its own thread
// (n_items <= NT): returns n_active; position_of(j) is then this thread's
// item's list position (active items ascending at [0, n_active), sinks
// ascending after them), valid when threadIdx.x < n_items.  Ends with a
// workgroup barrier.
template <int NT>
__device__ inline int32_t partition_one_pass(const uint8_t* s_sink, int32_t n_items, int32_t* s_wa,
                                             int32_t* s_ws, int32_t& pos) {
    constexpr int NWV = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t j = threadIdx.x;
    const bool in = j < n_items;
    const bool is_a = in && !s_sink[j];
    const uint64_t ba = __ballot(is_a), bs = __ballot(in && !is_a);
    if (lane == 0) {
        s_wa[wave] = __popcll(ba);
        s_ws[wave] = __popcll(bs);
    }
    __syncthreads();
    int32_t n_act = 0, pa = 0, ps = 0;
    for (int w = 0; w < NWV; ++w) {
        n_act += s_wa[w];
        if (w < wave) {
            pa += s_wa[w];
            ps += s_ws[w];
        }
    }
    pos = is_a ? pa + __popcll(ba & lt) : n_act + ps + __popcll(bs & lt);
    return n_act;
}

// Stable partition of the items: active ones in ascending order at list
// positions [0, n_act), sinks in ascending order at [n_act, n_items).
// visit(pos, j) is called once for every item by the thread that owns it.
template <int NT, typename Visit>
__device__ inline void partition_items(const uint8_t* s_sink, int32_t n_items, int32_t n_act,
                                       int32_t* s_wa, int32_t* s_ws, Visit visit) {
    constexpr int NWV = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t base_a = 0, base_s = n_act;
    for (int32_t c0 = 0; c0 < n_items; c0 += NT) {
        const int32_t j = c0 + threadIdx.x;
        const bool in = j < n_items;
        const bool is_a = in && !s_sink[j];
        const bool is_s = in && s_sink[j];
        const uint64_t ba = __ballot(is_a), bs = __ballot(is_s);
        if (lane == 0) {
            s_wa[wave] = __popcll(ba);
            s_ws[wave] = __popcll(bs);
        }
        __syncthreads();
        int32_t pa = base_a, ps = base_s, ta = 0, ts = 0;
        for (int w = 0; w < NWV; ++w) {
            if (w < wave) {
                pa += s_wa[w];
                ps += s_ws[w];
            }
            ta += s_wa[w];
            ts += s_ws[w];
        }
        if (is_a) visit(pa + __popcll(ba & lt), j);
        if (is_s) visit(ps + __popcll(bs & lt), j);
        base_a += ta;
        base_s += ts;
        __syncthreads();
    }
}

}  // namespace sr

namespace sr {

// A value every lane holds alike, moved to a scalar register: values read
// from LDS or memory are otherwise assumed to differ per lane, and the work
// division derived from them would live in vector registers behind
// per-lane branches.
__device__ inline int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline int64_t uniform64(int64_t x) {
    const uint64_t u = static_cast<uint64_t>(x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The plan's fields in scalar registers (integer division runs on the vector
// unit).
__device__ inline SplitPlan uniform_plan(SplitPlan p) {
    p.A = uniform64(p.A);
    p.e = uniform(p.e);
    p.C = uniform(p.C);
    p.n = uniform(p.n);
    p.S = uniform(p.S);
    p.P = uniform(p.P);
    p.Q = uniform(p.Q);
    p.rem = uniform(p.rem);
    p.balanced = uniform(p.balanced);
    return p;
}

template <int D, int NT, int CHUNK>
__device__ inline bool map_work(const DecodeArgs& a, WorkRange& r) {
    const int32_t n_items = a.batch * a.num_kv_heads;
    const int32_t wg = blockIdx.x;
    const int32_t G = a.group;
    int32_t n_act, sink_item = -1;
    r.item[0] = r.item[1] = -1;
    // The plan, this workgroup's range of positions and the list positions
    // of the items it touches (one in lanes mode, at most two when balanced).
    auto plan_range = [&](int32_t n) {
        r.plan = uniform_plan(
            make_split_plan(a.fixed_splits, a.grid, a.split_cap, n, a.seq_len, CHUNK));
        r.w = wg;
        r.i_begin = r.i_end = 0;
        r.lane = 0;
        r.p0 = r.p1 = 0;
        if (wg >= r.plan.P) return;
        if (!r.plan.balanced) {  // lane wg mod S of item wg / S
            r.i_begin = uniform(wg / r.plan.S);
            r.i_end = r.i_begin + 1;
            r.lane = wg - r.i_begin * r.plan.S;
            return;
        }
        r.p0 = uniform64(range_begin(r.plan, wg));
        r.p1 = uniform64(range_begin(r.plan, wg + 1));
        range_items(r.plan, wg, r.i_begin, r.i_end);
        r.i_begin = uniform(r.i_begin);
        r.i_end = uniform(r.i_end);
    };
    if (a.fused) {
        // the host runs fused routing only for n_items <= B*Hq <= kMaxFusedHeads <= NT:
        // every item has a thread and one ballot pass partitions them
        static_assert(kMaxFusedHeads <= NT, "one-pass partition needs a thread per item");
        __shared__ uint8_t s_flag[kMaxFusedHeads];
        __shared__ int32_t s_wa[NT / 64], s_ws[NT / 64];
        __shared__ int32_t s_pick[3];  // items at positions i_begin, i_begin + 1; the sink
        const bool w0 = wg == 0;
        if (threadIdx.x < 3) s_pick[threadIdx.x] = -1;
        route_items<NT, 8>(a.q, a.k0, a.tau, n_items, G, D, s_flag, w0 ? a.scores_out : nullptr,
                           w0 ? a.mask_out : nullptr);
        int32_t* list = w0 ? a.list_out : nullptr;
        int32_t pos;
        n_act = uniform(partition_one_pass<NT>(s_flag, n_items, s_wa, s_ws, pos));
        plan_range(n_act);
        const int32_t j = threadIdx.x;
        if (j < n_items) {
            if (pos == r.i_begin && pos < r.i_end) s_pick[0] = j;
            if (pos == r.i_begin + 1 && pos < r.i_end) s_pick[1] = j;
            if (pos == n_act + wg) s_pick[2] = j;
            if (list) list[pos] = j;
        }
        __syncthreads();
        if (w0 && threadIdx.x == 0 && a.n_active_out) a.n_active_out[0] = n_act;
        r.item[0] = uniform(s_pick[0]);
        r.item[1] = uniform(s_pick[1]);
        sink_item = uniform(s_pick[2]);
    } else if (a.routed && n_items <= NT) {
        // one round trip: the whole list and n_active load together
        __shared__ int32_t s_list[NT];
        __shared__ int32_t s_nact;
        if (static_cast<int32_t>(threadIdx.x) < n_items) s_list[threadIdx.x] = a.work_list[threadIdx.x];
        if (threadIdx.x == 0) s_nact = *a.n_active;
        __syncthreads();
        n_act = uniform(min(max(s_nact, 0), n_items));
        plan_range(n_act);
        if (n_act + wg < n_items) sink_item = uniform(s_list[n_act + wg]);
        if (r.i_begin < r.i_end) r.item[0] = uniform(s_list[r.i_begin]);
        if (r.i_begin + 1 < r.i_end) r.item[1] = uniform(s_list[r.i_begin + 1]);
    } else {
        n_act = a.routed ? uniform(min(max(*a.n_active, 0), n_items)) : n_items;
        plan_range(n_act);
        if (a.routed && n_act + wg < n_items) sink_item = uniform(a.work_list[n_act + wg]);
        if (r.i_begin < r.i_end) r.item[0] = a.routed ? uniform(a.work_list[r.i_begin]) : r.i_begin;
        if (r.i_begin + 1 < r.i_end)
            r.item[1] = a.routed ? uniform(a.work_list[r.i_begin + 1]) : r.i_begin + 1;
    }
    if (sink_item >= 0) {
        const int32_t b = sink_item / a.num_kv_heads, g = sink_item - b * a.num_kv_heads;
        const float* src = a.v0 + static_cast<int64_t>(sink_item) * D;
        float* dst =
            a.out + (static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(g) * G) * D;
        for (int x = threadIdx.x; x < G * D; x += NT) dst[x] = src[x % D];
    }
    return r.i_begin < r.i_end;
}

}  // namespace sr
