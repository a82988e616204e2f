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

#include <type_traits>

#include "decode_common.h"
#include "rope.h"

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
        // a zero vector scores 0; a non-finite input leaves a NaN, which fails
        // every threshold (the head dissents)
        c[r] = den != 0.f ? dot / den : 0.f;
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
            const float c = den != 0.f ? dot / den : 0.f;  // as head_cosines16
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

// The fused prologue's decisions for a layer of at most 64 items (B*Hq
// heads of G per item, at most 64), by NT threads: returns the 64-bit mask of
// sink items (bit j set: every head of item j has cos >= tau), the same in
// every wave.  Lane group k of wave w scores heads base + 4w + k + r*GROUPS,
// so one ballot per round gives the wave four consecutive heads' pass bits;
// each wave keeps a 64-bit mask of its heads' passes, leaves it in
// s_bits[wave], and after one barrier every thread ORs the NT/64 masks and
// lane j tests item j's G bits; a ballot gathers the items.  Scores are
// written when `scores` is non-null.
template <int NT, int U>
__device__ __attribute__((always_inline)) inline uint64_t fused_sink_mask(const float* __restrict__ q,
                                           const float* __restrict__ k0, float tau,
                                           int32_t n_items, int32_t G, int32_t d,
                                           uint64_t* s_bits, float* scores) {
    constexpr int GROUPS = NT / 16, NW = NT / 64;
    const int tid = threadIdx.x, hl = tid & 15, hg = tid >> 4, lane = tid & 63, wave = tid >> 6;
    const int32_t n_heads = n_items * G;
    uint64_t mine = 0;  // pass bits of the heads this wave scored (the same in every lane)
    // Each lane group takes heads hg, hg + GROUPS, ...; a round issues the
    // loads of only as many head slots as the round has live (1, 2, 4 or U),
    // since every slot's loads go out unconditionally.
    auto round = [&](auto slots, int32_t base, int32_t n_live) {
        constexpr int V = decltype(slots)::value;
        float c[V];
        head_cosines16<V>(q, k0, base + hg, GROUPS, n_heads, G, d, hl, n_live, c);
#pragma unroll
        for (int r = 0; r < V; ++r) {
            const int32_t hh = base + hg + r * GROUPS;
            if (scores && hh < n_heads && hl == 0) scores[hh] = c[r];
            // lanes 0, 16, 32, 48 hold heads first .. first + 3; NaN fails: the head dissents
            const uint64_t b = __ballot(hl == 0 && hh < n_heads && c[r] >= tau);
            const uint64_t nib = (b & 1u) | ((b >> 15) & 2u) | ((b >> 30) & 4u) | ((b >> 45) & 8u);
            const int32_t first = base + 4 * wave + r * GROUPS;
            if (first < 64) mine |= nib << first;
        }
    };
    for (int32_t base = 0; base < n_heads; base += GROUPS * U) {
        const int32_t n_live = (n_heads - base + GROUPS - 1) / GROUPS;  // same for every thread
        if (n_live <= 1) round(std::integral_constant<int, 1>{}, base, n_live);
        else if (n_live <= 2 && U > 2) round(std::integral_constant<int, 2>{}, base, n_live);
        else if (n_live <= 4 && U > 4) round(std::integral_constant<int, 4>{}, base, n_live);
        else round(std::integral_constant<int, U>{}, base, n_live);
    }
    if (lane == 0) s_bits[wave] = mine;
    __syncthreads();
    uint64_t heads = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) heads |= s_bits[w];
    const uint64_t gmask = (G >= 64 ? 0ull : (1ull << G)) - 1ull;  // G <= 16
    const int32_t at = lane < n_items ? lane * G : 0;
    const bool sink = lane < n_items && ((heads >> at) & gmask) == gmask;
    return __ballot(sink);
}

// Position of the k-th set bit (k = 0 for the lowest) of m, or -1.
__device__ inline int32_t nth_set_bit(uint64_t m, int32_t k) {
    for (; k > 0 && m; --k) m &= m - 1;
    return m ? static_cast<int32_t>(__builtin_ctzll(m)) : -1;
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

// Fused rotary, first step: every workgroup turns all B*Hq new queries to
// position T - 1 (the new token's) in LDS; workgroup 0 also writes them out.
// Each thread loads its query pairs first, so that their loads are in
// flight while the angles are computed.  The angles' cosines and sines stay
// in LDS for the key rows.  (Copying k0 to LDS here as well, to save the
// scores' own load, measured slower: the scores are bound by their
// arithmetic, and the rotation then waits for more loads.)
template <int D, int NT>
__device__ inline const float* rope_queries(const DecodeArgs& a, double*& s_c, double*& s_s) {
    extern __shared__ float4 s_rope[];  // rope_lds_bytes(B * Hq, D)
    constexpr int HALF = D / 2;
    constexpr int MAXP = (kMaxFusedHeads * HALF + NT - 1) / NT;  // pairs per thread
    s_c = reinterpret_cast<double*>(s_rope);
    s_s = s_c + HALF;
    float* s_q = reinterpret_cast<float*>(s_s + HALF);
    const int32_t n = a.batch * a.num_q_heads * HALF;
    float x0[MAXP], x1[MAXP];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {  // pairs past n read pair 0 and go unused
        const int32_t e = threadIdx.x + j * NT < n ? threadIdx.x + j * NT : 0;
        const int32_t row = e / HALF, i = e - row * HALF;
        x0[j] = a.q[static_cast<int64_t>(row) * D + i];
        x1[j] = a.q[static_cast<int64_t>(row) * D + i + HALF];
    }
    const int64_t pos = a.seq_len - 1;
    for (int i = threadIdx.x; i < HALF; i += NT) rope_angle(pos, a.inv_freq, i, s_c[i], s_s[i]);
    __syncthreads();
    const bool out = blockIdx.x == 0 && a.q_out;
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int32_t e = threadIdx.x + j * NT;
        if (e >= n) break;
        const int32_t row = e / HALF, i = e - row * HALF;
        double r0, r1;
        rope_turn(x0[j], x1[j], s_c[i], s_s[i], r0, r1);
        const float f0 = static_cast<float>(r0), f1 = static_cast<float>(r1);
        s_q[row * D + i] = f0;
        s_q[row * D + i + HALF] = f1;
        if (out) {
            a.q_out[static_cast<int64_t>(row) * D + i] = f0;
            a.q_out[static_cast<int64_t>(row) * D + i + HALF] = f1;
        }
    }
    __syncthreads();
    return s_q;
}

// Fused rotary, second step: the new key (turned) and value of item j go to
// row T - 1 of the caches, rounded as by the standalone rotary kernel.
template <int D, int NT>
__device__ inline void append_row(const DecodeArgs& a, int32_t j, const double* s_c,
                                  const double* s_s) {
    constexpr int HALF = D / 2;
    const int32_t b = j / a.num_kv_heads, g = j - b * a.num_kv_heads;
    const int64_t at = b * a.stride_b + g * a.stride_h + (a.seq_len - 1) * a.stride_t;
    const int32_t dtype = a.kv_f32 ? SR_KV_F32 : SR_KV_BF16;
    void* kc = const_cast<void*>(a.k);
    void* vc = const_cast<void*>(a.v);
    const float* kn = a.k_new + static_cast<int64_t>(j) * D;
    const float* vn = a.v_new + static_cast<int64_t>(j) * D;
    for (int i = threadIdx.x; i < HALF; i += NT) {
        double r0, r1;
        rope_turn(kn[i], kn[i + HALF], s_c[i], s_s[i], r0, r1);
        store_elem(kc, at + i, r0, dtype);
        store_elem(kc, at + i + HALF, r1, dtype);
        store_elem(vc, at + i, vn[i], dtype);
        store_elem(vc, at + i + HALF, vn[i + HALF], dtype);
    }
}

template <int D, int NT, int CHUNK>
__device__ inline bool map_work(const DecodeArgs& a, WorkRange& r) {
    const int32_t n_items = a.batch * a.num_kv_heads;
    const int32_t wg = blockIdx.x;
    const int32_t G = a.group;
    int32_t n_act, sink_item = -1;
    r.item[0] = r.item[1] = -1;
    r.q = a.q;
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
        // the host runs fused routing only for n_items <= B*Hq <= kMaxFusedHeads <= 64:
        // one ballot holds every item's decision, and the stable partition,
        // the count and the items this workgroup needs follow from it in
        // scalar registers, with no further barrier
        static_assert(kMaxFusedHeads <= 64, "one ballot covers every item");
        static_assert(kMaxFusedHeads <= 4 * (NT / 16), "one round of at most 4 heads per group");
        __shared__ uint64_t s_bits[NT / 64];
        const bool w0 = wg == 0;
        double *s_c = nullptr, *s_s = nullptr;
        if (a.rope) r.q = rope_queries<D, NT>(a, s_c, s_s);
        const uint64_t all = n_items >= 64 ? ~0ull : ((1ull << n_items) - 1);
        uint64_t sinks;
        if (a.flags_in) {  // decided by the routing kernel: every wave ballots the flags
            const int lane = threadIdx.x & 63;
            sinks = __ballot(lane < n_items && a.flags_in[lane] != 0) & all;
        } else {
            sinks = fused_sink_mask<NT, 4>(r.q, a.k0, a.tau, n_items, G, D, s_bits,
                                           w0 ? a.scores_out : nullptr) & all;
        }
        const uint64_t act = all & ~sinks;
        n_act = uniform(__popcll(act));
        plan_range(n_act);
        if (r.i_begin < r.i_end) r.item[0] = uniform(nth_set_bit(act, r.i_begin));
        if (r.i_begin + 1 < r.i_end) r.item[1] = uniform(nth_set_bit(act, r.i_begin + 1));
        if (n_act + wg < n_items) sink_item = uniform(nth_set_bit(sinks, wg));
        const int32_t j = threadIdx.x;
        if (w0 && j < n_items) {  // the routing outputs, from workgroup 0
            const bool is_sink = (sinks >> j) & 1ull;
            const uint64_t below = (1ull << j) - 1;
            const int32_t pos = is_sink ? n_act + __popcll(sinks & below) : __popcll(act & below);
            if (a.mask_out) a.mask_out[j] = is_sink ? 1 : 0;
            if (a.list_out) a.list_out[pos] = j;
            if (j == 0 && a.n_active_out) a.n_active_out[0] = n_act;
        }
        if (a.rope) {
            // Row T - 1 of every item is written by exactly one workgroup:
            // for a sink, the one that copies its v0 rows; for an active
            // item, the one whose part holds the chunk with T - 1, the only
            // workgroup that reads that row in this launch (the other parts'
            // prefetches past the end read row T - 2 instead: WorkUnit::clamp).
            // It writes before it streams, and its own loads then see the row.
            const SplitPlan& p = r.plan;
            const int32_t c = static_cast<int32_t>((a.seq_len - 1) / CHUNK);
            const int32_t l = c % p.S, k = c / p.S;  // lane and step of that chunk
            if (sink_item >= 0) append_row<D, NT>(a, sink_item, s_c, s_s);
            for (int32_t i = r.i_begin; i < r.i_end; ++i) {
                const int64_t x = static_cast<int64_t>(i) * p.C + lane_start(p, l) + k;
                const bool owner = p.balanced ? (r.p0 <= x && x < r.p1) : l == r.lane;
                if (owner) append_row<D, NT>(a, i == r.i_begin ? r.item[0] : r.item[1], s_c, s_s);
            }
            __builtin_amdgcn_s_waitcnt(0);  // the rows are in this XCD's L2
            __syncthreads();
        }
    } else if (a.routed && n_items <= NT) {
        // one round trip: the whole list and n_active load together
        __shared__ int32_t s_list[NT];
        __shared__ int32_t s_nact;
        // entries outside [0, B*Hkv) (a list not made by sr_route) are clamped
        // into range: wrong results, but no access outside the buffers
        if (static_cast<int32_t>(threadIdx.x) < n_items)
            s_list[threadIdx.x] = min(max(a.work_list[threadIdx.x], 0), n_items - 1);
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
        auto listed = [&](int32_t i) {  // clamped as above
            return uniform(min(max(a.work_list[i], 0), n_items - 1));
        };
        if (a.routed && n_act + wg < n_items) sink_item = listed(n_act + wg);
        if (r.i_begin < r.i_end) r.item[0] = a.routed ? listed(r.i_begin) : r.i_begin;
        if (r.i_begin + 1 < r.i_end)
            r.item[1] = a.routed ? listed(r.i_begin + 1) : r.i_begin + 1;
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
