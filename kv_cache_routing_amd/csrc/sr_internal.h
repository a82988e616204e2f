// Internal declarations shared by the libsinkroute translation units.
// Nothing here is part of the C ABI (that is include/sinkroute.h).
#pragma once

#include <hip/hip_runtime.h>
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
    float* part_ml;            // [grid][2][GP]   split maxima and sums
    float* part_acc;           // [grid][GP][d]   split accumulators
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
    float* alpha0_out;         // [B][Hq] weight of position 0 per head (optional)
};

// The fused route+decode prologue keeps one flag per item in LDS.
constexpr int32_t kMaxFusedItems = 4096;

// Adaptive mode never makes a split shorter than this many positions.
constexpr int64_t kMinSplitLen = 512;
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

inline int32_t pad_group(int32_t g) {
    int32_t p = 1;
    while (p < g) p <<= 1;
    return p;
}

// Host launchers, one per translation unit.
hipError_t launch_record(const sr_shape& s, const void* k, const void* v, float* k0, float* v0,
                         hipStream_t st);
hipError_t launch_route(const sr_shape& s, const float* q, const float* k0, float tau,
                        float* scores, uint8_t* mask, int32_t* work_list, int32_t* n_active,
                        hipStream_t st);
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
