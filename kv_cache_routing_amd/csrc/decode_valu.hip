// Split-K flash-decode of the active groups with vector-ALU dot products.
// Handles fp32 and bf16 caches, d in {64, 128}, any group size up to 16.
//
// Layout: a wave reads a tile of whole cache rows.  Each lane owns E = 8
// consecutive elements of one row (16 B of bf16, 32 B of fp32; E = 4, 8 B of
// bf16 or 16 B of fp32, for groups of 16 heads, whose query and accumulator
// rows would not fit the register file at 8), so a row is spread over d/E
// lanes (a "lane group")
// and one wave-wide load instruction covers 64/(d/E) consecutive rows: fully
// coalesced.  QK is an E-term dot product per lane followed by a DPP
// all-reduce inside the lane group; PV accumulates p * V for the lane's E
// elements.  Every lane group keeps its own
// running maximum, sum and accumulator (online softmax in base 2, rescaled
// only when a tile raises the maximum); the groups of a wave, then the waves
// of the workgroup, are merged at the end of the split.
//
// Method: SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time
// steps (tiled QK/PV with an online softmax, Split-K, in-kernel merge).
#include "routing.h"

namespace sr {
namespace {

// One lane's slice of a cache row: E consecutive elements, read with W
// non-temporal loads of type T and widened to fp32.
template <typename KV, int E>
struct RowSlice;

template <>
struct RowSlice<uint16_t, 8> {  // 8 bf16 in one 16-byte load
    using T = uint4;
    static constexpr int W = 1;
    __device__ static inline void load(T (&r)[W], const uint16_t* p) { r[0] = load_stream(p); }
    __device__ static inline void unpack(const T (&r)[W], float (&x)[8]) {
        const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

template <>
struct RowSlice<uint16_t, 4> {  // 4 bf16 in one 8-byte load
    using T = uint2;
    static constexpr int W = 1;
    __device__ static inline void load(T (&r)[W], const uint16_t* p) { r[0] = load_stream8(p); }
    __device__ static inline void unpack(const T (&r)[W], float (&x)[4]) {
        x[0] = __uint_as_float(r[0].x << 16);
        x[1] = __uint_as_float(r[0].x & 0xffff0000u);
        x[2] = __uint_as_float(r[0].y << 16);
        x[3] = __uint_as_float(r[0].y & 0xffff0000u);
    }
};

template <>
struct RowSlice<float, 8> {  // 8 fp32 in two 16-byte loads
    using T = uint4;
    static constexpr int W = 2;
    __device__ static inline void load(T (&r)[W], const float* p) {
        r[0] = load_stream(p);
        r[1] = load_stream(p + 4);
    }
    __device__ static inline void unpack(const T (&r)[W], float (&x)[8]) {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
    }
};

template <>
struct RowSlice<float, 4> {  // 4 fp32 in one 16-byte load
    using T = uint4;
    static constexpr int W = 1;
    __device__ static inline void load(T (&r)[W], const float* p) { r[0] = load_stream(p); }
    __device__ static inline void unpack(const T (&r)[W], float (&x)[4]) {
        x[0] = __uint_as_float(r[0].x);
        x[1] = __uint_as_float(r[0].y);
        x[2] = __uint_as_float(r[0].z);
        x[3] = __uint_as_float(r[0].w);
    }
};

template <typename KV, int D, int GP, int NW, int U, int E>
__global__ __launch_bounds__(NW * 64) void k_decode_valu(DecodeArgs a) {
    constexpr int LPT = D / E, TPI = 64 / LPT, TILE = TPI * U;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane / LPT, chunk = lane % LPT;

    __shared__ float s_m[NW][GP], s_l[NW][GP];
    __shared__ float s_acc[NW][GP][D];
    __shared__ float s_z0[GP];  // logits of position 0 (in the part that holds it)

    WorkRange wr;
    if (!map_work<D, NW * 64, NW * TILE>(a, wr)) return;
    const int32_t G = a.group;

    // One pass per item this workgroup has a part in: one, or two when the
    // work is balanced across an item boundary, the later item first (the
    // head of its first lane, read while the item's other workgroups are at
    // the same steps).  The pass is a lambda called at two sites rather than
    // a loop body, which keeps the register allocation of the common
    // one-pass case free of loop-carried state.  Merges that fall to this
    // workgroup run after the passes, when nothing else holds registers.
    auto pass = [&](int32_t part, MergeJob& job) -> bool {
        const WorkUnit u = part_of<NW * TILE>(a, wr, part);

        float qs[GP][E];
        {
            // branch-free loads, all issued before any is used: the padded
            // heads (h >= G) re-read the last real head and are zeroed by a
            // select (as loads under a branch, each waited for the one before)
            const float* qb = wr.q + (static_cast<int64_t>(u.b) * a.num_q_heads +
                                     static_cast<int64_t>(u.g) * G) * D + chunk * E;
            float4 xq[GP][E / 4];
#pragma unroll
            for (int h = 0; h < GP; ++h)
#pragma unroll
                for (int e4 = 0; e4 < E; e4 += 4)
                    xq[h][e4 / 4] = *reinterpret_cast<const float4*>(
                        qb + static_cast<int64_t>(h < G ? h : G - 1) * D + e4);
#pragma unroll
            for (int h = 0; h < GP; ++h)
#pragma unroll
                for (int e4 = 0; e4 < E; e4 += 4) {
                    const float4 x = xq[h][e4 / 4];
                    qs[h][e4] = h < G ? x.x * a.qscale : 0.f;
                    qs[h][e4 + 1] = h < G ? x.y * a.qscale : 0.f;
                    qs[h][e4 + 2] = h < G ? x.z * a.qscale : 0.f;
                    qs[h][e4 + 3] = h < G ? x.w * a.qscale : 0.f;
                }
        }

        const KV* kb = static_cast<const KV*>(a.k) + u.b * a.stride_b + u.g * a.stride_h + chunk * E;
        const KV* vb = static_cast<const KV*>(a.v) + u.b * a.stride_b + u.g * a.stride_h + chunk * E;
        const int64_t st = a.stride_t;

        float m[GP], l[GP], acc[GP][E];
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            m[h] = kNegInf;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
        }

        // One tile of TILE rows: the raw E-element slices this lane loads.
        using Slice = RowSlice<KV, E>;
        struct Raw {
            typename Slice::T k[U][Slice::W];
            typename Slice::T v[U][Slice::W];
        };
        const int64_t last = u.clamp;
        // Rows past T are clamped to one row (u.clamp): every lane then reads the
        // same row, so a prefetch past the end costs one row and no branch.
        auto issue = [&](Raw& r, int64_t tile) {
#pragma unroll
            for (int v = 0; v < U; ++v) {
                int64_t t = tile + v * TPI + row;
                t = t < u.t1 ? t : last;
                Slice::load(r.k[v], kb + t * st);
                Slice::load(r.v[v], vb + t * st);
            }
        };
        auto compute = [&](const Raw& r, int64_t tile) {
            float z[U][GP];
#pragma unroll
            for (int v = 0; v < U; ++v) {
                float kf[E];
                Slice::unpack(r.k[v], kf);
                const bool valid = tile + v * TPI + row < u.t1;
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) s += qs[h][e] * kf[e];
                    s = group_allreduce_sum<LPT>(s);
                    z[v][h] = valid ? s : kNegInf;
                }
            }
            if (tile == 0 && row == 0 && chunk == 0) {  // position 0 is row 0 of tile 0
#pragma unroll
                for (int h = 0; h < GP; ++h) s_z0[h] = z[0][h];
            }
            bool up = false;
            float zm[GP];
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                zm[h] = z[0][h];
#pragma unroll
                for (int v = 1; v < U; ++v) zm[h] = fmaxf(zm[h], z[v][h]);
                up = up || (zm[h] > m[h]);
            }
            if (__any(up)) {
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const float mn = fmaxf(m[h], zm[h]);
                    const float al = mn > m[h] ? fast_exp2(m[h] - mn) : 1.f;
                    m[h] = mn;
                    l[h] *= al;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] *= al;
                }
            }
#pragma unroll
            for (int v = 0; v < U; ++v) {
                float vf[E];
                Slice::unpack(r.v[v], vf);
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const float p = z[v][h] == kNegInf ? 0.f : fast_exp2(z[v][h] - m[h]);
                    l[h] += p;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] += p * vf[e];
                }
            }
        };

        // Two-stage register pipeline over this part's chunks: the next tile's
        // loads are in flight while the current tile is computed.
        Raw ra, rb;
        stream_walk<TILE>(u.walk, wave, ra, rb, issue, compute);

        // merge the lane groups of this wave (lanes with the same chunk)
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                const float mo = __shfl_xor(m[h], o);
                const float lo = __shfl_xor(l[h], o);
                const float M = fmaxf(m[h], mo);
                const float wa = merge_weight(m[h], M), wb = merge_weight(mo, M);
                l[h] = l[h] * wa + lo * wb;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float ao = __shfl_xor(acc[h][e], o);
                    acc[h][e] = acc[h][e] * wa + ao * wb;
                }
                m[h] = M;
            }
        }
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
#pragma unroll
                for (int e = 0; e < E; ++e) s_acc[wave][h][chunk * E + e] = acc[h][e];
                if (chunk == 0) {
                    s_m[wave][h] = m[h];
                    s_l[wave][h] = l[h];
                }
            }
        }
        __syncthreads();
        job = merge_job(u);
        return finish_part<D, GP, NW>(a, u, s_m, s_l, s_acc, s_z0);
    };
    MergeJob job0{}, job1{};
    const bool owe1 = pass(wr.i_end - 1, job1);
    bool owe0 = false;
    if (wr.i_end - wr.i_begin == 2) {
        __syncthreads();  // the first pass is done with LDS
        owe0 = pass(wr.i_begin, job0);
    }
    for (int j = 0; j < 2; ++j) {
        if (!(j == 0 ? owe0 : owe1)) continue;
        __syncthreads();
        MergeJob job;
        job.slot = j == 0 ? job0.slot : job1.slot;
        job.b = j == 0 ? job0.b : job1.b;
        job.g = j == 0 ? job0.g : job1.g;
        job.parts = j == 0 ? job0.parts : job1.parts;
        job.base = j == 0 ? job0.base : job1.base;
        merge_item<D, GP, NW>(a, job);
    }
}

template <typename KV, int D, int GP, int NW>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
    constexpr int U = valu_rows_per_lane(GP, static_cast<int>(sizeof(KV)), NW);
    constexpr int E = valu_elems_per_lane(GP, static_cast<int>(sizeof(KV)));
    const size_t lds = a.rope ? rope_lds_bytes(a.batch * a.num_q_heads, D) : 0;
    hipLaunchKernelGGL((k_decode_valu<KV, D, GP, NW, U, E>), dim3(a.grid), dim3(NW * 64), lds, st,
                       a);
    return hipGetLastError();
}

template <typename KV, int D, int NW>
hipError_t launch_g(const DecodeArgs& a, int gp, hipStream_t st) {
    switch (gp) {
        case 1: return launch_t<KV, D, 1, NW>(a, st);
        case 2: return launch_t<KV, D, 2, NW>(a, st);
        case 4: return launch_t<KV, D, 4, NW>(a, st);
        case 8: return launch_t<KV, D, 8, NW>(a, st);
        case 16:  // four-wave workgroups only (make_plan)
            if constexpr (NW == 4) return launch_t<KV, D, 16, NW>(a, st);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <typename KV, int NW>
hipError_t launch_d(const sr_shape& s, const DecodeArgs& a, int gp, hipStream_t st) {
    return s.head_dim == 128 ? launch_g<KV, 128, NW>(a, gp, st) : launch_g<KV, 64, NW>(a, gp, st);
}

}  // namespace

hipError_t launch_decode_valu(const sr_shape& s, const DecodeArgs& a, int gp, int waves,
                              hipStream_t st) {
    if (s.kv_dtype == SR_KV_BF16)
        return waves == 8 ? launch_d<uint16_t, 8>(s, a, gp, st) : launch_d<uint16_t, 4>(s, a, gp, st);
    return waves == 8 ? launch_d<float, 8>(s, a, gp, st) : launch_d<float, 4>(s, a, gp, st);
}

}  // namespace sr
