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

// One 16-byte load of cache data with the non-temporal cache policy.  Every
// cache byte is read once per launch, so nothing is gained by keeping it in
// L2 or the Infinity Cache; on MI355X this policy streams measurably faster
// than the default one (about 7.3 vs 6.4 TB/s with the read probe).
__device__ inline uint4 load_stream(const void* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// The same for 8 bytes.
__device__ inline uint2 load_stream8(const void* p) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
    return make_uint2(t.x, t.y);
}

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

// Sum over aligned groups of N lanes (N in 4, 8, 16, 32) with DPP (and one
// lane swap across rows for 32); every lane of a group ends with the group's
// total.  All 64 lanes must be active.
template <int N>
__device__ inline float group_allreduce_sum(float x) {
    x += dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                          // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
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

// The chunks of one item that one workgroup takes (lane-major positions
// [q0, q1) of the item, see SplitPlan), visited lane by lane from the last
// lane of the range to the first, each lane with rising step k.  A range that
// ends at the head of one lane and starts in the tail of the previous one
// thus reads its head piece first: every workgroup of an item then moves
// through the steps k together, and the item's workgroups stream one window
// of the cache (DRAM pages stay open) rather than distant ranges.
// The walk keeps pos, the first cache position of the current chunk; within
// a lane it advances by step = S * chunk positions and is recomputed only at
// a lane change.  A finished walk points at `past` (>= T), where every row a
// prefetch asks for clamps to one cached row (WorkUnit::clamp).  Steps are 32-bit
// (C < 2^31), so the walk stays in scalar registers (the scalar unit has no
// 64-bit ordered compare).
struct ChunkWalk {
    int64_t pos, step, chunk, past;
    int32_t k, k_end, k_first;
    int32_t l, l_first, S, Q, rem;
    bool done;

    __device__ void next() {
        if (++k < k_end) {
            pos += step;
            return;
        }
        if (l == l_first) {
            done = true;
            pos = past;
            return;
        }
        --l;
        k = l == l_first ? k_first : 0;
        k_end = Q + (l < rem ? 1 : 0);
        pos = (l + static_cast<int64_t>(k) * S) * chunk;
    }
};

__device__ inline ChunkWalk make_walk(const SplitPlan& p, int64_t q0, int64_t q1, int32_t chunk,
                                      int64_t seq_len) {
    ChunkWalk c{};
    c.S = p.S;
    c.Q = p.Q;
    c.rem = p.rem;
    c.chunk = chunk;
    c.step = static_cast<int64_t>(p.S) * chunk;
    c.past = seq_len;
    c.pos = seq_len;
    c.done = q0 >= q1;
    if (c.done) return c;
    int32_t la, lb, ka, kb;
    lane_of(p, static_cast<int32_t>(q0), la, ka);
    lane_of(p, static_cast<int32_t>(q1 - 1), lb, kb);
    // Integer division runs on the vector unit; readfirstlane moves the
    // (workgroup-uniform) results back to scalar registers for the loop.
    c.l = __builtin_amdgcn_readfirstlane(lb);
    c.l_first = __builtin_amdgcn_readfirstlane(la);
    c.k_first = __builtin_amdgcn_readfirstlane(ka);
    c.k = c.l == c.l_first ? c.k_first : 0;
    c.k_end = __builtin_amdgcn_readfirstlane(kb + 1);
    c.pos = (c.l + static_cast<int64_t>(c.k) * c.S) * chunk;
    return c;
}

// One workgroup's part of one item: the item at work-list position `slot`,
// the chunks to stream, and where its partial result goes.
struct WorkUnit {
    int32_t slot;   // list position of the item (index of its ticket)
    int32_t b, g;
    int32_t parts;  // workgroups sharing the item (1: this one writes the output)
    int32_t base;   // partial slot of the item's first part
    int32_t mine;   // partial slot of this part
    int64_t t1;     // positions [0, t1) exist (t1 = T)
    int64_t clamp;  // the row a prefetch of a position >= T reads instead
    ChunkWalk walk;
};

// What the merge of an item needs (a workgroup may owe two merges).
struct MergeJob {
    int32_t slot, b, g, parts, base;
};

__device__ inline MergeJob merge_job(const WorkUnit& u) {
    return MergeJob{u.slot, u.b, u.g, u.parts, u.base};
}

// A workgroup's share of the launch: the split plan, its range of positions
// and the items (b * Hkv + g) at list positions i_begin .. i_end - 1.
struct WorkRange {
    SplitPlan plan;
    int64_t p0, p1;
    int32_t w, i_begin, i_end;
    int32_t lane;  // lanes mode: the one lane this workgroup streams
    int32_t item[2];
    const float* q;  // the queries the passes read (a.q, or rotated in LDS)
};

// Routing decision and work division of one workgroup, then its sink duty.
// Workgroup w copies v0 into the G output rows of the sink at list position
// n_active + w (if there is one), then takes its range of the split plan.
// Without routing the list is the identity; with sr_route the list and
// n_active come from device memory; in fused mode every workgroup derives
// the decisions itself (the same arithmetic as sr_route, so every workgroup
// agrees) and workgroup 0 writes the routing outputs.  Returns false when
// the workgroup has no part.  In lanes mode a lane with no chunk below T
// (S > C) is an empty part and still merges.
template <int D, int NT, int CHUNK>
__device__ inline bool map_work(const DecodeArgs& a, WorkRange& r);

// Part i (a list position in [r.i_begin, r.i_end)) of the workgroup's range;
// chunks of CHUNK positions.
template <int CHUNK>
__device__ inline WorkUnit part_of(const DecodeArgs& a, const WorkRange& r, int32_t i) {
    WorkUnit u;
    const SplitPlan& p = r.plan;
    const int32_t item = i == r.i_begin ? r.item[0] : r.item[1];
    u.slot = i;
    u.b = item / a.num_kv_heads;
    u.g = item - u.b * a.num_kv_heads;
    u.mine = r.w + i;
    u.t1 = a.seq_len;
    // A prefetch past the end reads one real row and discards it.  With the
    // rotary step fused, row T - 1 is written in this launch by the workgroup
    // that owns it, so the others must not read it: they take row T - 2
    // (T >= 2 there), which no workgroup writes.
    u.clamp = a.rope ? a.seq_len - 2 : a.seq_len - 1;
    if (!p.balanced) {  // all of lane r.lane: no division needed
        u.parts = p.S;
        u.base = i * p.S + i;
        ChunkWalk& c = u.walk;
        c = ChunkWalk{};
        c.S = p.S;
        c.Q = p.Q;
        c.rem = p.rem;
        c.chunk = CHUNK;
        c.step = static_cast<int64_t>(p.S) * CHUNK;
        c.past = a.seq_len;
        c.l = c.l_first = r.lane;
        c.k = c.k_first = 0;
        c.k_end = p.Q + (r.lane < p.rem ? 1 : 0);
        c.done = c.k_end == 0;
        c.pos = c.done ? c.past : static_cast<int64_t>(r.lane) * CHUNK;
        return u;
    }
    int32_t w_lo;
    item_parts(p, i, w_lo, u.parts);
    u.base = w_lo + i;
    const int64_t x0 = static_cast<int64_t>(i) * p.C;
    const int64_t q0 = r.p0 > x0 ? r.p0 - x0 : 0;
    const int64_t q1 = r.p1 - x0 < p.C ? r.p1 - x0 : p.C;
    u.walk = make_walk(p, q0, q1, CHUNK, a.seq_len);
    return u;
}

// Two-stage register pipeline over a walk: the next tile's loads are in
// flight while the current tile is computed, also across the lanes of the
// walk.  This wave's tile of a chunk starts at pos + wave * WT.  issue() must
// clamp rows past T to WorkUnit::clamp: the prefetch after the last tile asks
// for rows at or past T, which costs one row.
template <int WT, typename Raw, typename Issue, typename Compute>
__device__ inline void stream_walk(ChunkWalk w, int wave, Raw& ra, Raw& rb, Issue issue,
                                   Compute compute) {
    const int64_t wofs = static_cast<int64_t>(wave) * WT;
    int64_t ta = w.pos + wofs;
    issue(ra, ta);
    while (!w.done) {
        ChunkWalk n1 = w;
        n1.next();
        const int64_t tb = n1.pos + wofs;
        issue(rb, tb);
        compute(ra, ta);
        if (n1.done) break;
        ChunkWalk n2 = n1;
        n2.next();
        const int64_t tc = n2.pos + wofs;
        issue(ra, tc);
        compute(rb, tb);
        if (n2.done) break;
        w = n2;
        ta = tc;
    }
}

// A store that is visible to every XCD once acknowledged (device-scope
// coherent: it is written through the local L2 instead of staying dirty).
__device__ inline void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Weight of position 0 in head h of the item: exp2(z0 - M) / L, with z0 the
// base-2 logit the kernel computed for position 0 and (M, L) the item's final
// maximum and sum (Eq. (1): alpha_0).
__device__ inline void write_alpha0(const DecodeArgs& a, int32_t b, int32_t g, int h, float z0,
                                    float M, float L) {
    if (h >= a.group) return;
    a.alpha0_out[static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(g) * a.group +
                 h] = fast_exp2(z0 - M) / L;
}

// Last-arriver merge of the S split partials of one item (all threads of the
// workgroup).  Order is fixed: the maxima M_h, then per split the weights
// w_s = exp2(m_s - M) into LDS, then the weighted accumulators.  When a
// partial has fewer float4 slots than the workgroup has threads, GROUPS
// thread groups take splits s = gi, gi + GROUPS, ... each in ascending order
// and the group sums are added in ascending gi; the sums L_h = sum_s w_s l_s
// and the maxima use one fixed shuffle + LDS tree.  Results are bitwise
// reproducible for a given split count.
//
// Latency: every global load is issued before anything waits.  Each thread
// first loads (m, l) of its (split, head) pair in every pass over the splits
// (up to MP passes, so up to MP * SP splits, in one run of loads), then the
// accumulators of the first CH splits; loads return in order, so the maxima
// wait only for the (m, l) loads while the accumulators stream in.  A merge
// of up to CH splits costs one memory round trip plus LDS work; each further
// CH splits cost one more round trip for their accumulators.
template <int D, int GP, int NW>
__device__ inline void merge_splits(const DecodeArgs& a, const MergeJob& u, float* out_item) {
    constexpr int NT = NW * 64;
    constexpr int NV = GP * D / 4;                 // float4 slots per partial
    constexpr int GROUPS = NV >= NT ? 1 : NT / NV;
    constexpr int SLOTS = NV >= NT ? NV / NT : 1;  // float4 slots per thread
    constexpr int PF = SLOTS >= 2 ? 16 : 32;       // splits prefetched per thread and slot
    constexpr int CH = PF * GROUPS;                // splits per chunk
    static_assert(CH == merge_round_splits(D, GP, NW), "the host sizes lanes by this round");
    constexpr int SP = NT / GP;                    // splits one pass over (m, l) covers
    constexpr int MP = 2;                          // (m, l) passes held in registers
    constexpr int WS = MP * SP > CH ? MP * SP : CH;  // weights LDS holds
    static_assert(NT % GP == 0 && NV % (NV >= NT ? NT : NV) == 0, "merge layout");
    static_assert(CH % SP == 0, "a chunk is whole (m, l) passes");
    __shared__ float s_red[NW][GP];
    __shared__ float s_M[GP], s_L[GP];
    __shared__ float s_w[WS][GP];
    __shared__ float4 s_grp[GROUPS][GROUPS > 1 ? NV : 1];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int32_t G = a.group;
    const int32_t S = u.parts;
    const float* ml0 = a.part_ml + static_cast<int64_t>(u.base) * 3 * GP;
    // Nothing is in flight here (the ticket waited for every memory operation),
    // but the compiler cannot see that through the passes' control flow: it
    // guarded the registers of the streaming loop's last prefetch with waits
    // placed between the loads below, which held half of the accumulator
    // loads back until (m, l) had arrived.  An explicit wait, free at run time,
    // clears that bookkeeping, so every load below goes out at once.
    __builtin_amdgcn_s_waitcnt(0);
    const float4* acc0 =
        reinterpret_cast<const float4*>(a.part_acc + static_cast<int64_t>(u.base) * GP * D);
    const int gi = GROUPS > 1 ? t / NV : 0;
    const int v0 = GROUPS > 1 ? t % NV : t;
    const int hm = t % GP, sm = t / GP;  // this thread's (head, split) in every (m, l) pass

    // (m, l) of splits sm, sm + SP, ... (the passes the split count has, at
    // most MP; the pass count is the same in every thread, so the branches
    // are uniform), z0 of split 0 (position 0's logit), then the accumulators
    // of the first chunk.  No load depends on a per-lane condition: indexes
    // past the last split are clamped to it and the values masked (weight 0),
    // so the loads form one straight run and each wait counts exactly the
    // loads it needs.
    const int np = (S + SP - 1) / SP;
    const bool in_regs = np <= MP;  // every split's weight fits in LDS at once
    float mv[MP], lv[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        mv[p] = kNegInf;
        lv[p] = 0.f;
        if (p < np) {
            const int s = sm + p * SP;
            const int64_t o = static_cast<int64_t>(s < S ? s : S - 1) * 3 * GP;
            mv[p] = ml0[o + hm];
            lv[p] = ml0[o + GP + hm];
        }
    }
    const float z0 = ml0[2 * GP + (t < G ? t : 0)];
    float4 pre[SLOTS][PF];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j)
#pragma unroll
            for (int k = 0; k < PF; ++k) {
                const int sp = c0 + gi + GROUPS * k;
                pre[j][k] = acc0[static_cast<int64_t>(sp < S ? sp : S - 1) * NV + v0 + j * NT];
            }
    };
    fetch(0);
#pragma unroll
    for (int p = 0; p < MP; ++p)
        if (sm + p * SP >= S) {
            mv[p] = kNegInf;
            lv[p] = 0.f;
        }

    // Sum (or max) over the threads that hold head hm: lanes l, l ^ GP, ...
    // within the wave, then the waves in ascending order.
    auto head_reduce = [&](float x, bool is_max, float* dst) {
        for (int o = GP; o < 64; o <<= 1) {
            const float y = __shfl_xor(x, o);
            x = is_max ? fmaxf(x, y) : x + y;
        }
        if (lane < GP) s_red[wave][lane] = x;
        __syncthreads();
        if (t < GP) {
            float r = s_red[0][t];
            for (int w = 1; w < NW; ++w) r = is_max ? fmaxf(r, s_red[w][t]) : r + s_red[w][t];
            dst[t] = r;
        }
        __syncthreads();
    };

    float mx = mv[0];
#pragma unroll
    for (int p = 1; p < MP; ++p) mx = fmaxf(mx, mv[p]);
    for (int s = sm + MP * SP; s < S; s += SP)
        mx = fmaxf(mx, ml0[static_cast<int64_t>(s) * 3 * GP + hm]);
    head_reduce(mx, true, s_M);
    const float M = s_M[hm];

    float4 acc[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    // The weights: all of them at once from the registers, or (more than MP
    // passes) chunk by chunk, reloading (m, l).  Either way each thread adds
    // its w_s l_s in ascending s.
    float lw = 0.f;
    if (in_regs) {
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int s = p * SP + sm;
            if (s < S) {
                const float w = merge_weight(mv[p], M);
                s_w[s][hm] = w;
                lw += w * lv[p];
            }
        }
        // The sums L_h now, while the accumulators are still arriving (its
        // barrier also publishes the weights).
        head_reduce(lw, false, s_L);
    }
    for (int c0 = 0; c0 < S; c0 += CH) {
        if (c0 > 0) fetch(c0);
        const int n = S - c0 < CH ? S - c0 : CH;
        if (!in_regs) {
#pragma unroll
            for (int p = 0; p < CH / SP; ++p) {
                const int s = p * SP + sm;  // split index within the chunk
                if (s < n) {
                    float m = mv[0], l = lv[0];
                    if (c0 + p > 0) {
                        const float* q = ml0 + static_cast<int64_t>(c0 + s) * 3 * GP;
                        m = q[hm];
                        l = q[GP + hm];
                    }
                    const float w = merge_weight(m, M);
                    s_w[s][hm] = w;
                    lw += w * l;
                }
            }
            __syncthreads();
        }
        const int wo = in_regs ? c0 : 0;  // where this chunk's weights sit in LDS
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int h = (4 * (v0 + j * NT)) / D;
            float4 r = acc[j];
#pragma unroll
            for (int k = 0; k < PF; ++k) {
                const int s = gi + GROUPS * k;  // splits past S carry zeros and weight 0
                const float w = s < n ? s_w[wo + s][h] : 0.f;
                r.x += w * pre[j][k].x;
                r.y += w * pre[j][k].y;
                r.z += w * pre[j][k].z;
                r.w += w * pre[j][k].w;
            }
            acc[j] = r;
        }
        if (!in_regs) __syncthreads();  // the next chunk rewrites the weights
    }
    if (!in_regs) head_reduce(lw, false, s_L);
    if (t < G && a.alpha0_out) write_alpha0(a, u.b, u.g, t, z0, s_M[t], s_L[t]);
    if constexpr (GROUPS > 1) {
        s_grp[gi][v0] = acc[0];
        __syncthreads();
        if (gi == 0 && 4 * v0 < G * D) {
            float4 r = s_grp[0][v0];
            for (int g = 1; g < GROUPS; ++g) {
                const float4 x = s_grp[g][v0];
                r.x += x.x;
                r.y += x.y;
                r.z += x.z;
                r.w += x.w;
            }
            const float L = s_L[(4 * v0) / D];
            *reinterpret_cast<float4*>(out_item + 4 * v0) =
                make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
        }
    } else {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int v = v0 + j * NT;
            if (4 * v < G * D) {
                const float L = s_L[(4 * v) / D];
                const float4 r = acc[j];
                *reinterpret_cast<float4*>(out_item + 4 * v) =
                    make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
            }
        }
    }
}

// Merge the per-wave states held in LDS (s_m/s_l [NW][GP], s_acc [NW][GP][DS],
// rows of D values at a stride of DS)
// into this workgroup's partial of the item.  When the workgroup is the
// item's only part the partial is final and goes straight to `out`;
// otherwise it is stored at slot u.mine with device-coherent stores and a
// ticket is taken.  Returns true (in every thread) when this workgroup drew
// the item's last ticket: it must then merge the item (merge_item), after
// an acquire that this function has already made.
template <int D, int GP, int NW, int DS = D>
__device__ inline bool finish_part(const DecodeArgs& a, const WorkUnit& u,
                                   const float (*s_m)[GP], const float (*s_l)[GP],
                                   const float (*s_acc)[GP][DS], const float* s_z0) {
    constexpr int NT = NW * 64;
    const int32_t G = a.group;
    if (u.parts == 1) {
        float* out_item = a.out + (static_cast<int64_t>(u.b) * a.num_q_heads +
                                   static_cast<int64_t>(u.g) * G) * D;
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
            if (i == 0 && a.alpha0_out) write_alpha0(a, u.b, u.g, h, s_z0[h], M, L);
        }
        return false;
    }

    float* pml = a.part_ml + static_cast<int64_t>(u.mine) * 3 * GP;
    float* pacc = a.part_acc + static_cast<int64_t>(u.mine) * GP * D;
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
        store_coherent(pacc + x, A);
        if (i == 0) {
            store_coherent(pml + h, M);
            store_coherent(pml + GP + h, L);
            store_coherent(pml + 2 * GP + h, s_z0[h]);  // meaningful in the part holding position 0
        }
    }

    // Publish the partial and take a ticket.  The partial went out with
    // device-coherent stores, which write through this XCD's L2; each wave
    // waits until its stores are acknowledged, then thread 0 moves the ticket.
    // An agent-scope release fence here would instead write back the whole
    // L2 of the XCD in every wave of every workgroup at the end of the launch
    // (measured ~10 us of tail).  Only the workgroup that draws the last
    // ticket pays for an acquire (an L2 invalidation) before it reads the
    // other partials.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0: stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.tickets + u.slot, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == static_cast<uint32_t>(u.parts - 1);
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(s_last) != 0;
}

// The merge of an item whose last ticket this workgroup drew: all its parts
// in ascending workgroup order, written to `out`; the ticket is left at zero
// for the next call.
template <int D, int GP, int NW>
__device__ inline void merge_item(const DecodeArgs& a, const MergeJob& u) {
    float* out_item = a.out + (static_cast<int64_t>(u.b) * a.num_q_heads +
                               static_cast<int64_t>(u.g) * a.group) * D;
    merge_splits<D, GP, NW>(a, u, out_item);
    if (threadIdx.x == 0) a.tickets[u.slot] = 0u;  // ready for the next call
}

}  // namespace sr
