// Split-K flash-decode of the active groups on the matrix cores.  bf16
// caches: v_mfma_f32_16x16x32_bf16 for QK; PV on the vector ALUs for groups of
// up to 4 heads, on v_mfma_f32_16x16x16_bf16 for 8 and 16.  fp32 caches: a
// second kernel below, QK and PV on v_mfma_f32_16x16x4_f32.
//
// A wave step covers one 16-position tile (two at d = 64, where one tile is
// only 4 KiB of bf16 keys and values: too little per wait to keep HBM busy);
// the next step's loads are in flight while the current one is computed.
//
// QK as a 16x16 tile product per 16 cache rows: the G query heads padded to
// 16 rows against 16 key rows (row of the cache), fp32 logits.  Lane l feeds
// key row (l mod 16) with the 8 bf16 at d = 32*kb + 8*(l/16) of k-block kb,
// so each load instruction takes 64 contiguous bytes of 16 rows.  The query
// is pre-scaled by sm_scale*log2(e) and split exactly enough into hi + lo
// bf16 terms (two MFMAs per k-block): products with the stored bf16 keys are
// exact and the logits carry ~2^-16 relative error in the query.
//
// Groups of up to 4 heads: queries are the A operand, so lane l holds heads
// 4*(l/16)..+3 of position (l mod 16) and the running maximum of a head is
// uniform across a 16-lane row (DPP row max, only when some logit exceeds
// it).  The probabilities go through LDS to the PV layout, where lane l owns
// 8 consecutive elements of one value row (16 B, coalesced 1 KiB per wave
// instruction) and accumulates p * V in fp32 for the group's heads.
//
// Groups of 8 or 16 heads, where p * V on the vector ALUs would bound the
// kernel (2*G*d flops per 4*d bytes): the keys are the A operand, so lane l
// holds head (l mod 16) at positions 4*(l/16)..+3.  That is the B operand
// layout of the PV product out^T[d][head] += V^T[d][pos] P^T[pos][head] on
// the 16x16x16 matrix cores, so the probabilities stay in registers (split
// into hi + lo bf16 terms like the query) and each head's maximum, sum and
// rescale live in its own lanes.  Only the value tile is transposed, through
// a padded per-wave LDS tile; the accumulator is D/16 fragments of 4 floats.
//
// Method: SinkRouter README (github.com/streamer-AP/SinkRouter), decode-time
// steps (tiled QK/PV with an online softmax, Split-K, in-kernel merge);
// result defined by Eq. (1) of the paper (pith.science, Figure 1 caption).
#include "routing.h"

namespace sr {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short bf16x4;  // bf16 bits, 16x16x16 operands
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ inline uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ inline float readlane_f(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

template <int D, int GP, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_mfma(DecodeArgs a) {
    constexpr int KB = D / 32;        // k-blocks of the QK product
    constexpr int LPT = D / 8;        // PV: lanes per value row
    constexpr int TPI = 64 / LPT;     // PV: rows per load instruction
    constexpr int UPS = 16 / TPI;     // PV: load instructions per 16 rows
    static_assert(GP <= 16, "at most 16 heads per group");
    constexpr int SUB = mfma_tiles_per_step(D, 2);  // 16-position tiles per wave step
    constexpr bool PVM = GP >= 8;     // PV on the matrix cores
    constexpr int DS = PVM ? D + 1 : D;  // s_acc row stride (odd: no bank conflicts)
    constexpr int VS = D + 4;         // s_v row stride in bf16 (264 / 136 B, 8-byte aligned)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;      // MFMA layout
    const int prow = lane / LPT, pchunk = lane % LPT;  // PV layout

    __shared__ __attribute__((aligned(16))) float s_p[NW][16][16];  // [pos][head]
    __shared__ float s_m[NW][GP], s_l[NW][GP];
    __shared__ float s_acc[NW][GP][DS];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[NW][PVM ? 16 : 1][PVM ? VS : 1];
    __shared__ float s_z0[GP];  // logits of position 0 (in the part that holds it)

    WorkRange wr;
    if (!map_work<D, NW * 64, NW * 16 * SUB>(a, wr)) return;
    const int32_t G = a.group;

    // One pass per item this workgroup has a part in: one, or two when the
    // work is balanced across an item boundary, the later item first (the
    // head of its first lane, read while the item's other workgroups are at
    // the same steps).  The pass is a lambda called at two sites rather than
    // a loop body, which keeps the register allocation of the common
    // one-pass case free of loop-carried state.  Merges that fall to this
    // workgroup run after the passes, when nothing else holds registers.
    auto pass = [&](int32_t part, MergeJob& job) -> bool {
        const WorkUnit u = part_of<NW * 16 * SUB>(a, wr, part);

        // A operands: query row = col, elements d = 32*kb + 8*grp + e.  Every
        // load goes out before any is used and none sits under a branch: the
        // padded rows (col >= G) read the group's last real row and are zeroed
        // by a select.  (q may be in memory or, with the rotary step fused, in
        // LDS, so these are generic loads; as loads under a per-lane condition
        // the compiler issued them one at a time, each waiting for the last:
        // about 2.5 us before the first cache load.)
        bf16x8 qhi[KB], qlo[KB];
        {
            const int32_t hq = col < G ? col : G - 1;
            const float* qr = wr.q + (static_cast<int64_t>(u.b) * a.num_q_heads +
                                     static_cast<int64_t>(u.g) * G + hq) * D + 8 * grp;
            const bool real = col < G;
            float4 xq[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                xq[kb][0] = *reinterpret_cast<const float4*>(qr + 32 * kb);
                xq[kb][1] = *reinterpret_cast<const float4*>(qr + 32 * kb + 4);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float xs[8] = {xq[kb][0].x, xq[kb][0].y, xq[kb][0].z, xq[kb][0].w,
                                     xq[kb][1].x, xq[kb][1].y, xq[kb][1].z, xq[kb][1].w};
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float x0 = real ? xs[e] * a.qscale : 0.f;
                    float x1 = real ? xs[e + 1] * a.qscale : 0.f;
                    const uint32_t h0 = bf16_rne_bits(x0), h1 = bf16_rne_bits(x1);
                    const uint32_t l0 = bf16_rne_bits(x0 - bf16_bits_to_float(h0));
                    const uint32_t l1 = bf16_rne_bits(x1 - bf16_bits_to_float(h1));
                    hw[e / 2] = h0 | (h1 << 16);
                    lw[e / 2] = l0 | (l1 << 16);
                }
                qhi[kb] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                qlo[kb] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
            }
        }

        const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + u.b * a.stride_b + u.g * a.stride_h;
        const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + u.b * a.stride_b + u.g * a.stride_h;
        const int64_t st = a.stride_t;

        // vector-ALU PV: m, lsum of heads 4*grp + i (uniform across the 16-lane
        // row) and acc[h][e] of value elements 8*pchunk + e.  Matrix-core PV:
        // m[0], lsum[0] of head col and accm[mb][i] = out^T[16*mb + 4*grp + i][col].
        float m[4], lsum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[i] = kNegInf;
            lsum[i] = 0.f;
        }
        float acc[PVM ? 1 : GP][8];
#pragma unroll
        for (int h = 0; h < (PVM ? 1 : GP); ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        f32x4 accm[PVM ? D / 16 : 1];
#pragma unroll
        for (int mb = 0; mb < (PVM ? D / 16 : 1); ++mb) accm[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

        // One 16-position tile: the raw key and value bytes this lane loads; a
        // wave step takes SUB of them.
        struct Tile16 {
            uint4 k[KB];
            uint4 v[UPS];
        };
        struct Raw {
            Tile16 t[SUB];
        };
        const int64_t last = u.clamp;
        // Positions past T are clamped to one row (u.clamp): every lane then reads
        // the same row, so a prefetch past the end costs one row and no branch.
        auto issue16 = [&](Tile16& r, int64_t tile) {
            int64_t tk = tile + col;
            tk = tk < u.t1 ? tk : last;
            const uint16_t* kp = kbase + tk * st + 8 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) r.k[kb] = load_stream(kp + 32 * kb);
#pragma unroll
            for (int uu = 0; uu < UPS; ++uu) {
                int64_t tv = tile + prow + TPI * uu;
                tv = tv < u.t1 ? tv : last;
                r.v[uu] = load_stream(vbase + tv * st + pchunk * 8);
            }
        };
        auto compute_pvm = [&](const Tile16& r, int64_t tile) {
            // logits with the keys as A: s[i] = head col at position tile + 4*grp + i
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 kv = __builtin_bit_cast(bf16x8, r.k[kb]);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qhi[kb], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[kb], s, 0, 0, 0);
            }
            // the tile's value rows into this wave's LDS tile, row-major
#pragma unroll
            for (int uu = 0; uu < UPS; ++uu) {
                uint2* dst = reinterpret_cast<uint2*>(&s_v[wave][prow + TPI * uu][pchunk * 8]);
                dst[0] = make_uint2(r.v[uu].x, r.v[uu].y);
                dst[1] = make_uint2(r.v[uu].z, r.v[uu].w);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)  // ragged tail: positions past T weigh nothing
                if (tile + 4 * grp + i >= u.t1) s[i] = kNegInf;
            if (tile == 0 && grp == 0 && col < GP) s_z0[col] = s[0];  // position 0
            float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (__any(mx > m[0])) {
                const float mn = fmaxf(m[0], mx);
                const float al = mn > m[0] ? fast_exp2(m[0] - mn) : 1.f;
                m[0] = mn;
                lsum[0] *= al;
#pragma unroll
                for (int mb = 0; mb < D / 16; ++mb) accm[mb] *= al;
            }
            bf16x4 phi, plo;  // P^T fragment, hi + lo bf16 terms
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = s[i] == kNegInf ? 0.f : fast_exp2(s[i] - m[0]);
                lsum[0] += p;
                const uint32_t h = bf16_rne_bits(p);
                phi[i] = static_cast<short>(h);
                plo[i] = static_cast<short>(bf16_rne_bits(p - bf16_bits_to_float(h)));
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int mb = 0; mb < D / 16; ++mb) {
                bf16x4 vt;  // V^T fragment: d = 16*mb + col at positions 4*grp + j
#pragma unroll
                for (int j = 0; j < 4; ++j) vt[j] = static_cast<short>(s_v[wave][4 * grp + j][16 * mb + col]);
                accm[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, accm[mb], 0, 0, 0);
                accm[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, accm[mb], 0, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
        };
        auto compute_valu = [&](const Tile16& r, int64_t tile) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 kv = __builtin_bit_cast(bf16x8, r.k[kb]);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[kb], kv, s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[kb], kv, s, 0, 0, 0);
            }
            if (tile + col >= u.t1) {  // ragged tail: positions past T weigh nothing
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = kNegInf;
            }
            if (tile == 0 && col == 0) {  // position 0 is column 0 of tile 0
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * grp + i < GP) s_z0[4 * grp + i] = s[i];
            }
            bool up = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) up = up || (s[i] > m[i]);
            if (__any(up)) {
                float alpha[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float mx = group_allreduce_max<16>(s[i]);
                    const float mn = fmaxf(m[i], mx);
                    alpha[i] = mn > m[i] ? fast_exp2(m[i] - mn) : 1.f;
                    m[i] = mn;
                    lsum[i] *= alpha[i];
                }
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const float al = readlane_f(alpha[h & 3], 16 * (h >> 2));
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] *= al;
                }
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = s[i] == kNegInf ? 0.f : fast_exp2(s[i] - m[i]);
                lsum[i] += p[i];
            }
            *reinterpret_cast<float4*>(&s_p[wave][col][4 * grp]) = make_float4(p[0], p[1], p[2], p[3]);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int uu = 0; uu < UPS; ++uu) {
                const int pos = prow + TPI * uu;
                float pr[GP];
                if constexpr (GP >= 4) {
#pragma unroll
                    for (int h4 = 0; h4 < GP; h4 += 4) {
                        const float4 x = *reinterpret_cast<const float4*>(&s_p[wave][pos][h4]);
                        pr[h4] = x.x;
                        pr[h4 + 1] = x.y;
                        pr[h4 + 2] = x.z;
                        pr[h4 + 3] = x.w;
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < GP; ++h) pr[h] = s_p[wave][pos][h];
                }
                const uint32_t w4[4] = {r.v[uu].x, r.v[uu].y, r.v[uu].z, r.v[uu].w};
                float vf[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vf[2 * i] = __uint_as_float(w4[i] << 16);
                    vf[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
                }
#pragma unroll
                for (int h = 0; h < GP; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] += pr[h] * vf[e];
            }
            __builtin_amdgcn_wave_barrier();
        };
        auto issue = [&](Raw& r, int64_t tile) {
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) issue16(r.t[sb], tile + 16 * sb);
        };
        auto compute = [&](const Raw& r, int64_t tile) {
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) {
                if constexpr (PVM) compute_pvm(r.t[sb], tile + 16 * sb);
                else compute_valu(r.t[sb], tile + 16 * sb);
            }
        };

        // Two-stage register pipeline over this part's chunks: the next tile's
        // loads are in flight while the current tile is computed.
        Raw ra, rb;
        stream_walk<16 * SUB>(u.walk, wave, ra, rb, issue, compute);

        if constexpr (PVM) {
            // head col's sum over the wave's positions (the four lane rows)
            lsum[0] += __shfl_xor(lsum[0], 16);
            lsum[0] += __shfl_xor(lsum[0], 32);
            if (col < GP) {
#pragma unroll
                for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s_acc[wave][col][16 * mb + 4 * grp + i] = accm[mb][i];
                if (grp == 0) {
                    s_m[wave][col] = m[0];
                    s_l[wave][col] = lsum[0];
                }
            }
        } else {
            // wave totals: sums over the 16 positions of a row, values over PV rows
#pragma unroll
            for (int i = 0; i < 4; ++i) lsum[i] = group_allreduce_sum<16>(lsum[i]);
#pragma unroll
            for (int o = LPT; o < 64; o <<= 1)
#pragma unroll
                for (int h = 0; h < GP; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
            if (prow == 0) {
#pragma unroll
                for (int h = 0; h < GP; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) s_acc[wave][h][pchunk * 8 + e] = acc[h][e];
            }
            if (col == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int h = 4 * grp + i;
                    if (h < GP) {
                        s_m[wave][h] = m[i];
                        s_l[wave][h] = lsum[i];
                    }
                }
            }
        }
        __syncthreads();
        job = merge_job(u);
        return finish_part<D, GP, NW, DS>(a, u, s_m, s_l, s_acc, s_z0);
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

// fp32 caches on the matrix cores: QK and PV on v_mfma_f32_16x16x4_f32, in
// fp32 throughout.  That instruction takes one value per lane (K = 4 across
// the four 16-lane rows), so the order in which d is contracted or produced
// is free, and it is chosen for contiguous 16-byte loads:
//   QK step kb (d/4 steps): lane (col, grp) feeds key row `col` and query head
//     `col` at element 16*(kb/4) + 4*grp + kb%4 (per row, the four lane rows
//     read 64 contiguous bytes per load instruction); the result holds head
//     `col` at positions 4*grp + i, as in the bf16 kernel's groups of 8 and 16.
//   PV step (kq, mb): position 4*grp + kq, output element
//     4*m + 64*(mb/4) + mb%4 of row m = col (16 lanes read a whole 256-byte
//     stretch of a value row per instruction); the probability is the lane's
//     own p[kq], so nothing goes through LDS.
// Every group size pads to 16 heads; partials, merge and work division are
// the bf16 kernel's.
template <int D, int GP, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_mfma_f32(DecodeArgs a) {
    constexpr int KD = D / 4;   // QK steps
    constexpr int DV = D / 16;  // PV output blocks
    constexpr int DS = D + 1;   // s_acc row stride (odd: no bank conflicts)
    static_assert(GP <= 16, "at most 16 heads per group");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;

    __shared__ float s_m[NW][GP], s_l[NW][GP];
    __shared__ float s_acc[NW][GP][DS];
    __shared__ float s_z0[GP];

    WorkRange wr;
    if (!map_work<D, NW * 64, NW * 16>(a, wr)) return;
    const int32_t G = a.group;

    auto pass = [&](int32_t part, MergeJob& job) -> bool {
        const WorkUnit u = part_of<NW * 16>(a, wr, part);

        float qv[KD];  // B operand of QK: head col, element 16*(kb/4) + 4*grp + kb%4
        {
            // branch-free loads, all issued before any is used (padded rows
            // re-read the last real row and are zeroed by the select)
            const int32_t hq = col < G ? col : G - 1;
            const float* qr = wr.q + (static_cast<int64_t>(u.b) * a.num_q_heads +
                                     static_cast<int64_t>(u.g) * G + hq) * D + 4 * grp;
            const float sc = col < G ? a.qscale : 0.f;
            float4 xq[KD / 4];
#pragma unroll
            for (int j = 0; j < KD / 4; ++j) xq[j] = *reinterpret_cast<const float4*>(qr + 16 * j);
#pragma unroll
            for (int j = 0; j < KD / 4; ++j) {
                const float4 x = xq[j];
                qv[4 * j] = col < G ? x.x * sc : 0.f;
                qv[4 * j + 1] = col < G ? x.y * sc : 0.f;
                qv[4 * j + 2] = col < G ? x.z * sc : 0.f;
                qv[4 * j + 3] = col < G ? x.w * sc : 0.f;
            }
        }
        const float* kbase = static_cast<const float*>(a.k) + u.b * a.stride_b + u.g * a.stride_h;
        const float* vbase = static_cast<const float*>(a.v) + u.b * a.stride_b + u.g * a.stride_h;
        const int64_t st = a.stride_t;

        float m = kNegInf, lsum = 0.f;  // head col
        f32x4 accm[DV];                 // out[col][4*(4*grp + i) + 64*(mb/4) + mb%4]
#pragma unroll
        for (int mb = 0; mb < DV; ++mb) accm[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

        struct Raw {
            uint4 k[KD / 4];      // key row tile + col, elements 16*j + 4*grp ..
            uint4 v[4][DV / 4];   // value rows tile + 4*grp + kq, elements 4*col + 64*h ..
        };
        const int64_t last = u.clamp;
        // Rows past T are clamped to one row (u.clamp): a prefetch past the end
        // costs one row and no branch.
        auto issue = [&](Raw& r, int64_t tile) {
            int64_t tk = tile + col;
            tk = tk < u.t1 ? tk : last;
            const float* kp = kbase + tk * st + 4 * grp;
#pragma unroll
            for (int j = 0; j < KD / 4; ++j) r.k[j] = load_stream(kp + 16 * j);
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                int64_t tv = tile + 4 * grp + kq;
                tv = tv < u.t1 ? tv : last;
                const float* vp = vbase + tv * st + 4 * col;
#pragma unroll
                for (int h = 0; h < DV / 4; ++h) r.v[kq][h] = load_stream(vp + 64 * h);
            }
        };
        auto compute = [&](const Raw& r, int64_t tile) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KD / 4; ++j) {
                const uint4 k = r.k[j];
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.x), qv[4 * j], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.y), qv[4 * j + 1], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.z), qv[4 * j + 2], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w), qv[4 * j + 3], s, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)  // ragged tail: positions past T weigh nothing
                if (tile + 4 * grp + i >= u.t1) s[i] = kNegInf;
            if (tile == 0 && grp == 0 && col < GP) s_z0[col] = s[0];  // position 0
            float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (__any(mx > m)) {
                const float mn = fmaxf(m, mx);
                const float al = mn > m ? fast_exp2(m - mn) : 1.f;
                m = mn;
                lsum *= al;
#pragma unroll
                for (int mb = 0; mb < DV; ++mb) accm[mb] *= al;
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = s[i] == kNegInf ? 0.f : fast_exp2(s[i] - m);
                lsum += p[i];
            }
#pragma unroll
            for (int kq = 0; kq < 4; ++kq)
#pragma unroll
                for (int h = 0; h < DV / 4; ++h) {
                    const uint4 v = r.v[kq][h];
                    accm[4 * h] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), p[kq], accm[4 * h], 0, 0, 0);
                    accm[4 * h + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), p[kq], accm[4 * h + 1], 0, 0, 0);
                    accm[4 * h + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), p[kq], accm[4 * h + 2], 0, 0, 0);
                    accm[4 * h + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), p[kq], accm[4 * h + 3], 0, 0, 0);
                }
        };

        Raw ra, rb;
        stream_walk<16>(u.walk, wave, ra, rb, issue, compute);

        lsum += __shfl_xor(lsum, 16);  // head col's sum over the wave's positions
        lsum += __shfl_xor(lsum, 32);
        if (col < GP) {
#pragma unroll
            for (int mb = 0; mb < DV; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_acc[wave][col][4 * (4 * grp + i) + 64 * (mb >> 2) + (mb & 3)] = accm[mb][i];
            if (grp == 0) {
                s_m[wave][col] = m;
                s_l[wave][col] = lsum;
            }
        }
        __syncthreads();
        job = merge_job(u);
        return finish_part<D, GP, NW, DS>(a, u, s_m, s_l, s_acc, s_z0);
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

template <bool F32, int D, int GP, int NW>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
    const size_t lds = a.rope ? rope_lds_bytes(a.batch * a.num_q_heads, D) : 0;
    if constexpr (F32)
        hipLaunchKernelGGL((k_decode_mfma_f32<D, GP, NW>), dim3(a.grid), dim3(NW * 64), lds, st, a);
    else
        hipLaunchKernelGGL((k_decode_mfma<D, GP, NW>), dim3(a.grid), dim3(NW * 64), lds, st, a);
    return hipGetLastError();
}

template <bool F32, int D, int NW>
hipError_t launch_g(const DecodeArgs& a, int gp, hipStream_t st) {
    switch (gp) {
        case 1: return launch_t<F32, D, 1, NW>(a, st);
        case 2: return launch_t<F32, D, 2, NW>(a, st);
        case 4: return launch_t<F32, D, 4, NW>(a, st);
        case 8: return launch_t<F32, D, 8, NW>(a, st);
        case 16: return launch_t<F32, D, 16, NW>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool F32>
hipError_t launch_w(const sr_shape& s, const DecodeArgs& a, int gp, int waves, hipStream_t st) {
    if (waves == 8)
        return s.head_dim == 128 ? launch_g<F32, 128, 8>(a, gp, st) : launch_g<F32, 64, 8>(a, gp, st);
    return s.head_dim == 128 ? launch_g<F32, 128, 4>(a, gp, st) : launch_g<F32, 64, 4>(a, gp, st);
}

}  // namespace

hipError_t launch_decode_mfma(const sr_shape& s, const DecodeArgs& a, int gp, int waves,
                              hipStream_t st) {
    return s.kv_dtype == SR_KV_F32 ? launch_w<true>(s, a, gp, waves, st)
                                   : launch_w<false>(s, a, gp, waves, st);
}

}  // namespace sr
