// Measurement helper: a read-only HBM streaming kernel with the same access
// width as the decode kernels (16 bytes per lane per load), used to measure
// the achievable read bandwidth ceiling the decode kernels are compared with.
#include "sr_internal.h"

namespace sr {
namespace {

// blocked = 0: the grid walks the buffer together (workgroup w reads chunks
// w, w + grid, ...); blocked = 1: workgroup w streams its own contiguous
// slice of bytes / grid, the access shape of one decode split.  NTL selects
// the non-temporal cache policy for the loads.
template <int U, bool NTL>
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     int32_t blocked,
                                                     uint32_t* __restrict__ sink) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    uint32_t x = 0;
    int64_t begin = static_cast<int64_t>(blockIdx.x) * 256 * U;
    int64_t step = static_cast<int64_t>(gridDim.x) * 256 * U;
    int64_t end = n16;
    if (blocked) {
        const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
        begin = static_cast<int64_t>(blockIdx.x) * per;
        end = begin + per < n16 ? begin + per : n16;
        step = 256 * U;
    }
    for (int64_t base = begin; base < end; base += step) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i >= end) {
                v[u] = make_uint4(0, 0, 0, 0);
            } else if (NTL) {
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
                v[u] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
                v[u] = p[i];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // The data decide whether anything is stored, so no load can be dropped;
    // for real data the store practically never happens.
    if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// One 16-byte direct-to-LDS load per lane: lane l's 16 bytes land at
// dst + 16 * l (dst is the wave's tile, the same in every lane).  The
// builtin exists only for the GPU; the host pass of this file, which never
// runs it, must not see it (it would drop the kernels' launch stubs).
__device__ inline void load_to_lds16(const uint4* src, uint4* dst, bool nontemporal) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (nontemporal)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);  // nt
    else
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}

// The same walk with the loads staged through LDS: each wave's loads go
// straight from memory into its LDS tile (global_load_lds_dwordx4, 1 KiB per
// wave and instruction, no register holds the data in flight), then every
// lane reads its 16 bytes back.  Lanes past the end load the last 16 bytes
// again (no branch around the DMA).  This is the access shape of a decode
// kernel that stages K/V tiles in LDS; comparing it with k_stream_read shows
// whether staging reads faster.
template <int U, bool NTL>
__global__ __launch_bounds__(256) void k_stream_read_lds(const uint4* __restrict__ p, int64_t n16,
                                                         int32_t blocked,
                                                         uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint4 tile[4][U][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = 0;
    int64_t begin = static_cast<int64_t>(blockIdx.x) * 256 * U;
    int64_t step = static_cast<int64_t>(gridDim.x) * 256 * U;
    int64_t end = n16;
    if (blocked) {
        const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
        begin = static_cast<int64_t>(blockIdx.x) * per;
        end = begin + per < n16 ? begin + per : n16;
        step = 256 * U;
    }
    for (int64_t base = begin; base < end; base += step) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t i = base + u * 256 + threadIdx.x;
            i = i < end ? i : end - 1;
            load_to_lds16(p + i, &tile[wave][u][0], NTL);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the DMA writes to LDS have landed
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint4 v = tile[wave][u][lane];
            x ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

template <bool NTL>
hipError_t launch_lds(const uint4* p, int64_t n16, int32_t grid, int32_t unroll, int32_t blocked,
                      uint32_t* sink, hipStream_t st) {
    switch (unroll) {
        case 1: hipLaunchKernelGGL((k_stream_read_lds<1, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 2: hipLaunchKernelGGL((k_stream_read_lds<2, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 4: hipLaunchKernelGGL((k_stream_read_lds<4, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 8: hipLaunchKernelGGL((k_stream_read_lds<8, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 16: hipLaunchKernelGGL((k_stream_read_lds<16, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool NTL>
hipError_t launch_policy(const uint4* p, int64_t n16, int32_t grid, int32_t unroll,
                         int32_t blocked, uint32_t* sink, hipStream_t st) {
    switch (unroll) {
        case 1: hipLaunchKernelGGL((k_stream_read<1, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 2: hipLaunchKernelGGL((k_stream_read<2, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 4: hipLaunchKernelGGL((k_stream_read<4, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 8: hipLaunchKernelGGL((k_stream_read<8, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        case 16: hipLaunchKernelGGL((k_stream_read<16, NTL>), dim3(grid), dim3(256), 0, st, p, n16, blocked, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, int32_t grid, int32_t unroll,
                              int32_t flags, uint32_t* sink, hipStream_t st) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const auto* p = static_cast<const uint4*>(buf);
    const int32_t blocked = flags & SR_READ_BLOCKED;
    if (flags & SR_READ_LDS)
        return (flags & SR_READ_NONTEMPORAL)
                   ? launch_lds<true>(p, n16, grid, unroll, blocked, sink, st)
                   : launch_lds<false>(p, n16, grid, unroll, blocked, sink, st);
    return (flags & SR_READ_NONTEMPORAL)
               ? launch_policy<true>(p, n16, grid, unroll, blocked, sink, st)
               : launch_policy<false>(p, n16, grid, unroll, blocked, sink, st);
}

}  // namespace sr
