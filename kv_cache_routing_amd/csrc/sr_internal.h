// Internal declarations shared by the libsinkroute translation units.
// Nothing here is part of the C ABI (that is include/sinkroute.h).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sinkroute.h"

namespace sr {

// Launch-time description of one decode call, passed by value to the kernels.
struct DecodeArgs {
    const float* q;            // [B][Hq][d] fp32
    const void* k;             // cache base (bf16 or fp32 elements)
    const void* v;
    const float* v0;           // [B][Hkv][d] fp32 (routed only)
    const int32_t* work_list;  // [B*Hkv] (routed only)
    const int32_t* n_active;   // [1]     (routed only)
    float* out;                // [B][Hq][d] fp32
    uint32_t* tickets;         // [B*Hkv] arrival counters, zero between calls
    float* part_ml;            // [grid + B*Hkv][3][GP]  part maxima, sums, position-0 logits
    float* part_acc;           // [grid + B*Hkv][GP][d]  part accumulators
    int64_t stride_b, stride_h, stride_t;  // elements
    int64_t seq_len;
    int32_t batch, num_q_heads, num_kv_heads, group;
    float qscale;              // sm_scale * log2(e): logits are kept in base 2
    int32_t fixed_splits;      // > 0: fixed split count; 0: adaptive
    int32_t grid;              // workgroups launched
    int32_t split_cap;         // adaptive: upper bound on splits per item
    int32_t routed;            // v0 is valid; sinks are bypassed
    // Fused routing (sr_route_decode): every workgroup derives the routing
    // decision from q and k0 itself; workgroup 0 also writes the optional
    // routing outputs.  When 0, work_list / n_active come from sr_route.
    int32_t fused;
    const float* k0;           // [B][Hkv][d] fp32 (fused only)
    float tau;
    float* scores_out;         // [B][Hq]   (fused, optional)
    uint8_t* mask_out;         // [B][Hkv]  (fused, optional)
    int32_t* list_out;         // [B*Hkv]   (fused, optional)
    int32_t* n_active_out;     // [1]       (fused, optional)
    // Fused, from flags: the routing kernel scored every group and wrote one
    // flag byte per item (B*Hkv <= 64); the decode workgroups take the
    // decisions from there instead of scoring (flags_in == nullptr: score).
    const uint8_t* flags_in;
    float* alpha0_out;         // [B][Hq] weight of position 0 per head (optional)
    // Fused rotary + append (sr_rope_route_decode, fused routing only): q is
    // the unrotated new query; every workgroup rotates all queries to
    // position T - 1 into dynamic LDS (rope_lds_bytes), and the key and value
    // rows at T - 1 are written by the one workgroup that reads them.
    int32_t rope;
    int32_t kv_f32;            // cache elements are fp32 (else bf16)
    const float* k_new;        // [B][Hkv][d] fp32, unrotated (rope only)
    const float* v_new;        // [B][Hkv][d] fp32 (rope only)
    const float* inv_freq;     // [d/2] (rope only)
    float* q_out;              // [B][Hq][d] rotated query (rope, optional)
};

// Dynamic LDS of a fused rotary launch: cos and sin of the d/2 angles (fp64),
// then the rotated queries [B*Hq][d] fp32 (16-byte aligned).
__host__ __device__ constexpr size_t rope_lds_bytes(int32_t q_rows, int32_t d) {
    return static_cast<size_t>(d / 2) * 2 * sizeof(double) +
           static_cast<size_t>(q_rows) * d * sizeof(float);
}

// sr_route_decode runs routing inside the decode launch (every workgroup
// scores every head) only for layers of up to this many query heads; larger
// layers run the routing kernel and then the decode, which measured faster
// (a prologue that scores 128 heads per workgroup already costs more than
// the extra launch).  The fused prologue keeps one pass bit per head in a
// 64-bit mask and partitions the items in one ballot pass, so it needs
// items <= heads <= 64.
constexpr int32_t kMaxFusedHeads = 64;

// Most workgroups the routing kernel spreads its scoring over.
constexpr int32_t kRouteMaxWgs = 1024;

// Launch defaults: wave64s per decode workgroup and workgroups per CU in
// the adaptive grid.
constexpr int kDefaultWaves = 4;
constexpr int kDefaultWgsPerCu = 1;

// Splits per active item; the kernels and the host use this same function.
__host__ __device__ inline int32_t splits_for(int32_t fixed_splits, int32_t grid,
                                              int32_t split_cap, int32_t n_act) {
    if (fixed_splits > 0) return fixed_splits;
    if (n_act <= 0) return 1;
    int32_t s = grid / n_act;
    if (s > split_cap) s = split_cap;
    return s < 1 ? 1 : s;
}

// Work division of a decode launch (the kernels and the host share it).
//
// Each active item's cache is cut into C = ceil(T / chunk) chunks of `chunk`
// positions (one tile per wave).  The chunks of an item are ordered
// lane-major: lane l (of S lanes) holds chunks l, l + S, l + 2S, ..., and the
// lanes follow each other; the n active items' sequences are concatenated in
// work-list order, N = n * C positions in all.  Workgroup w takes the
// positions [begin(w), begin(w + 1)):
//
// * lanes mode (the S lanes of every item fill the grid, a fixed split count
//   was asked for, or the split cap is reached): exactly lane w mod S of
//   item w / S, so the workgroups of an item stream one interleaved window;
// * balanced mode (the lanes leave workgroups over, e.g. 29 items on 256
//   workgroups): an equal share floor(w N / P) .. floor((w + 1) N / P), so no
//   CU idles; a share is at most C positions, so it touches at most two items.
//
// Workgroup w's work on item i is one "part"; the parts of an item are the
// workgroups w_lo(i) .. w_hi(i) and their partial results sit at slots
// w + i, contiguous per item (w + i is injective over the parts).
struct SplitPlan {
    int64_t A;         // balanced: floor(N / P), positions per workgroup
    int32_t C;         // chunks per item (< 2^31)
    int32_t e;         // balanced: N mod P
    int32_t n;         // active items
    int32_t S;         // lanes per item
    int32_t P;         // workgroups with cache work
    int32_t Q, rem;    // lane l holds Q + (l < rem) chunks
    int32_t balanced;
};

// Balanced mode keeps products like w * n and w * (N mod P) below 2^30.
constexpr int32_t kMaxBalancedGrid = 1 << 15;

// Everything below runs in 32-bit arithmetic (N = n * C can exceed 2^32,
// but no 64-bit division is needed): with C = c1 * P + c2,
// floor(N / P) = n * c1 + floor(n * c2 / P), and n * c2 < 2^30.
__host__ __device__ inline SplitPlan make_split_plan(int32_t fixed_splits, int32_t grid,
                                                     int32_t split_cap, int32_t n_act,
                                                     int64_t seq_len, int32_t chunk) {
    SplitPlan p{};
    p.n = n_act > 0 ? n_act : 0;
    p.C = static_cast<int32_t>((seq_len + chunk - 1) / chunk);
    p.S = splits_for(fixed_splits, grid, split_cap, n_act);
    p.Q = p.C / p.S;
    p.rem = p.C - p.Q * p.S;
    p.balanced = fixed_splits == 0 && p.n > 0 && p.S < split_cap &&
                 static_cast<int64_t>(p.n) * p.S < grid && grid <= kMaxBalancedGrid;
    p.P = p.balanced ? grid : p.n * p.S;
    if (p.balanced) {
        const int32_t c1 = p.C / p.P, c2 = p.C - c1 * p.P;
        const int32_t nc2 = p.n * c2;
        p.A = static_cast<int64_t>(p.n) * c1 + nc2 / p.P;
        p.e = nc2 - (nc2 / p.P) * p.P;
    }
    return p;
}

__host__ __device__ inline int32_t lane_start(const SplitPlan& p, int32_t l) {
    return l * p.Q + (l < p.rem ? l : p.rem);
}

// Lane and step of lane-major position q (0 <= q < C) of an item.
__host__ __device__ inline void lane_of(const SplitPlan& p, int32_t q, int32_t& l, int32_t& k) {
    const int32_t big = p.rem * (p.Q + 1);
    if (q < big) {
        l = q / (p.Q + 1);
        k = q - l * (p.Q + 1);
    } else {  // here Q >= 1: with Q == 0 every position lies below `big`
        const int32_t r = q - big;
        l = p.rem + r / p.Q;
        k = r - (l - p.rem) * p.Q;
    }
}

// First position of workgroup w's range (w <= P; begin(P) = N).
__host__ __device__ inline int64_t range_begin(const SplitPlan& p, int32_t w) {
    if (p.balanced) return static_cast<int64_t>(w) * p.A + (w * p.e) / p.P;  // floor(w N / P)
    return static_cast<int64_t>(w / p.S) * p.C + lane_start(p, w % p.S);
}

// List positions of the items workgroup w (< P) has parts in: [i_begin, i_end).
__host__ __device__ inline void range_items(const SplitPlan& p, int32_t w, int32_t& i_begin,
                                            int32_t& i_end) {
    if (!p.balanced) {
        i_begin = w / p.S;
        i_end = i_begin + 1;
        return;
    }
    i_begin = (w * p.n) / p.P;  // floor(floor(w N / P) / C) = floor(w n / P)
    // a range is at most C long (P >= n), so it reaches at most one more item
    i_end = range_begin(p, w + 1) > static_cast<int64_t>(i_begin + 1) * p.C ? i_begin + 2
                                                                           : i_begin + 1;
}

// The workgroup holding position x = i * C, the first of item i (i <= n;
// item n stands for the end, P): the largest w with begin(w) <= x, which is
// floor(i P / n) or one more.
__host__ __device__ inline int32_t item_first_wg(const SplitPlan& p, int32_t i) {
    if (i >= p.n) return p.P;
    const int32_t m = (i * p.P) / p.n;
    return range_begin(p, m + 1) <= static_cast<int64_t>(i) * p.C ? m + 1 : m;
}

// The parts of item i: first workgroup and count.
__host__ __device__ inline void item_parts(const SplitPlan& p, int32_t i, int32_t& w_lo,
                                           int32_t& parts) {
    if (!p.balanced) {
        w_lo = i * p.S;
        parts = p.S;
        return;
    }
    w_lo = item_first_wg(p, i);
    // the last part is the workgroup holding (i + 1) C - 1: the first
    // workgroup of item i + 1, unless that one starts exactly at its start
    const int32_t w_next = item_first_wg(p, i + 1);
    const bool starts_there =
        w_next >= p.P || range_begin(p, w_next) == static_cast<int64_t>(i + 1) * p.C;
    parts = (starts_there ? w_next - 1 : w_next) - w_lo + 1;
}

// Elements of a cache row per lane (E), rows of cache per lane and tile (U)
// of the vector-ALU kernel, and the positions per chunk of either kernel.
// Sized so that nothing spills: a lane holds its query and accumulator rows
// (2 x GP x E floats) and two tiles of U slices of K and V.  fp32 rows take
// two 16-byte loads per 8 elements, so they get half the rows.  Groups of 16
// heads take 4 elements per lane (8-byte bf16 slices) and always run in
// four-wave workgroups (make_plan): with two waves per SIMD, 256 registers
// each, their state does not fit at any tile size.  Eight-wave workgroups of
// 4-head bf16 groups take half the rows.
__host__ __device__ constexpr int valu_elems_per_lane(int gp, int kv_bytes) {
    return gp >= 16 ? 4 : 8;
}

__host__ __device__ constexpr int valu_rows_per_lane(int gp, int kv_bytes, int waves) {
    const int u = valu_elems_per_lane(gp, kv_bytes) == 4
                      ? 4
                      : (gp >= 8 ? 2 : (kv_bytes == 4 ? 4 : 8));
    return waves == 8 && gp == 4 && kv_bytes == 2 ? u / 2 : u;
}

// 16-position tiles per wave step of the matrix-core kernels: bf16 rows of
// d = 64 are 256 bytes, and one tile per step left the loads too short to
// keep HBM busy (two: 5.7 -> 6.7 TB/s at G = 8; at d = 128 one is best).
__host__ __device__ constexpr int mfma_tiles_per_step(int head_dim, int kv_bytes) {
    return kv_bytes == 2 && head_dim == 64 ? 2 : 1;
}

inline int32_t chunk_positions(int32_t kernel, int32_t head_dim, int32_t gp, int32_t waves,
                               int32_t kv_bytes) {
    if (kernel == SR_KERNEL_MFMA) return waves * 16 * mfma_tiles_per_step(head_dim, kv_bytes);
    return waves * (64 / (head_dim / valu_elems_per_lane(gp, kv_bytes))) *
           valu_rows_per_lane(gp, kv_bytes, waves);
}

inline int32_t pad_group(int32_t g) {
    int32_t p = 1;
    while (p < g) p <<= 1;
    return p;
}

// Splits the last-arriver merge takes per memory round trip (merge_splits:
// each thread holds PF accumulator slots of one split group in registers).
constexpr int32_t merge_round_splits(int32_t d, int32_t gp, int32_t waves) {
    const int32_t nt = waves * 64, nv = gp * d / 4;
    const int32_t groups = nv >= nt ? 1 : nt / nv;
    const int32_t slots = nv >= nt ? nv / nt : 1;
    return (slots >= 2 ? 16 : 32) * groups;
}

// Adaptive mode's cap on lanes per item.  More lanes cut the chunks each
// part streams; past a multiple of merge_round_splits they add a round trip
// to the item's merge, which the last part to arrive runs alone.  Measured on
// MI355X (sweeps of the lane count at 4K to 512K positions, one to four
// active items, groups of 2 to 8 heads): a part streams a chunk at about
// 36 GB/s, and each merge round costs about 3 us (its round trip plus the
// partials through one CU).  The cap is the lane count S that minimises
// ceil(C / S) chunk times plus ceil(S / round) round times, over the best
// S of each round count (S = min(C, grid, rounds * round)); ties keep fewer
// rounds.
inline int32_t adaptive_split_cap(int64_t seq_len, int32_t chunk, int64_t chunk_bytes,
                                  int32_t round, int32_t grid) {
    constexpr double kChunkBytesPerUs = 36.0e3;  // one part's streaming rate
    constexpr double kRoundUs = 3.0;             // one merge round
    const int64_t chunks = (seq_len + chunk - 1) / chunk;
    const int64_t top = chunks < grid ? chunks : grid;
    if (top <= 1) return 1;
    // The continuous optimum is near r* = sqrt(C * chunk time / (round * round
    // time)); round counts up to about twice that cover the discrete one and
    // keep the search short on huge grids and caches.
    const double chunk_us = static_cast<double>(chunk_bytes) / kChunkBytesPerUs;
    const int64_t r_max = 2 + static_cast<int64_t>(
        2.0 * sqrt(static_cast<double>(chunks) * chunk_us / (static_cast<double>(round) * kRoundUs)));
    int64_t best_s = 1;
    double best = 0.0;
    for (int64_t r = 1; r <= r_max; ++r) {
        const int64_t s = r * round < top ? r * round : top;
        const double cost = static_cast<double>((chunks + s - 1) / s) * chunk_us +
                            kRoundUs * static_cast<double>(r);
        if (r == 1 || cost < best) {
            best = cost;
            best_s = s;
        }
        if (s == top) break;
    }
    return static_cast<int32_t>(best_s);
}

// Host launchers, one per translation unit.
hipError_t launch_record(const sr_shape& s, const void* k, const void* v, float* k0, float* v0,
                         hipStream_t st);
// ticket: a zeroed counter in device memory, or null (a second launch then
// partitions large layers).
// The rotary step done by the routing kernel (sr_rope_route_decode on layers
// above kMaxFusedHeads query heads): the workgroup that scores an item first
// turns its heads' new queries to position pos into q_out and appends its
// new key and value row there; the scores are then taken from q_out.
// q_new == nullptr: no rotary step (q is already rotated).
struct RouteRope {
    const float* q_new;     // [B][Hq][d] unrotated
    const float* k_new;     // [B][Hkv][d] unrotated
    const float* v_new;     // [B][Hkv][d]
    const float* inv_freq;  // [d/2]
    float* q_out;           // [B][Hq][d] rotated (required)
    void* k_cache;
    void* v_cache;
    int64_t stride_b, stride_h, stride_t, pos;
    int32_t kv_f32;
};

hipError_t launch_route(const sr_shape& s, const float* q, const float* k0, float tau,
                        float* scores, uint8_t* flags, int32_t* work_list, int32_t* n_active,
                        uint32_t* ticket, hipStream_t st, const RouteRope& rope = RouteRope{});
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_rope_append(const sr_shape& s, const float* q_new, const float* k_new,
                              const float* v_new, const float* inv_freq, int64_t pos,
                              float* q_out, void* k_cache, void* v_cache, hipStream_t st);
hipError_t launch_decode_valu(const sr_shape& s, const DecodeArgs& a, int gp, int waves,
                              hipStream_t st);
hipError_t launch_decode_mfma(const sr_shape& s, const DecodeArgs& a, int gp, int waves,
                              hipStream_t st);
hipError_t launch_stream_read(const void* buf, size_t bytes, int32_t grid, int32_t unroll,
                              int32_t flags, uint32_t* sink, hipStream_t st);

}  // namespace sr
