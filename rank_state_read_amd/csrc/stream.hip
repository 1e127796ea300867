// Streaming probe for gfx950: the practical HBM rate of a plain stream with a
// chosen read:write mix, measured beside the decode kernels so that their
// achieved bandwidth can be stated against what this machine delivers for the
// same mix (the vendor's 8 TB/s is a peak no access pattern reaches).
//
// A chunk is unroll x 4 KB: thread t of a 256-thread block reads 16-byte
// pieces t, t + 256, ..., so each wave instruction covers 1 KB contiguous and
// each thread has `unroll` pieces in flight.  With a write ratio m the thread
// then stores, for every m pieces, their sum (a 16-byte piece) into the
// chunk's slice of dst (m is 1, 2, 4, 8 or 16 and divides `unroll`);
// read-only runs keep a running sum and store one piece per thread at the
// end.  The sums keep every load live.  Every access covers whole 128-byte
// lines, so the non-temporal variant loses no reuse; on MI355X it streamed
// ~15% faster than plain loads and stores.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "sketchssm_internal.h"
#include "sketchssm_measure.h"

namespace skssm {

template <bool NT>
__device__ __forceinline__ f32x4 stream_ld(const f32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void stream_st(f32x4 v, f32x4* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int U, int M, bool NT>
__global__ __launch_bounds__(256) void stream_kernel(const f32x4* __restrict__ src, size_t nchunks,
                                                     f32x4* __restrict__ dst) {
    const int t = threadIdx.x;
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const f32x4* p = src + c * (U * 256) + t;
        f32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = stream_ld<NT>(p + j * 256);
        if constexpr (M > 0) {
            f32x4* q = dst + c * size_t(U / M * 256) + t;
#pragma unroll
            for (int o = 0; o < U / M; ++o) {
                f32x4 s = v[o * M];
#pragma unroll
                for (int i = 1; i < M; ++i) s += v[o * M + i];
                stream_st<NT>(s, q + o * 256);
            }
        } else {
#pragma unroll
            for (int j = 0; j < U; ++j) tot += v[j];
        }
    }
    if constexpr (M == 0) dst[size_t(blockIdx.x) * 256 + t] = tot;
}

template <int U, bool NT>
static void launch_stream(int m, size_t grid, hipStream_t s, const f32x4* src, size_t nchunks, f32x4* dst) {
    switch (m) {
        case 0: hipLaunchKernelGGL((stream_kernel<U, 0, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst); break;
        case 1: hipLaunchKernelGGL((stream_kernel<U, 1, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst); break;
        case 2: hipLaunchKernelGGL((stream_kernel<U, 2, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst); break;
        case 4: hipLaunchKernelGGL((stream_kernel<U, 4, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst); break;
        default:
            if constexpr (U >= 8) {
                if (m == 8)
                    hipLaunchKernelGGL((stream_kernel<U, 8, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst);
            }
            if constexpr (U >= 16) {
                if (m == 16)
                    hipLaunchKernelGGL((stream_kernel<U, 16, NT>), dim3(grid), dim3(256), 0, s, src, nchunks, dst);
            }
            break;
    }
}

}  // namespace skssm

using namespace skssm;

extern "C" sketchssm_status sketchssm_stream_probe(const void* src, size_t read_bytes, void* dst,
                                                   size_t write_bytes, int32_t unroll, int32_t blocks,
                                                   int32_t flags, void* stream) {
    if (!src || !dst || blocks < 0 || (flags & ~1) != 0) return SKSSM_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return SKSSM_EALIGN;
    if (unroll != 4 && unroll != 8 && unroll != 16) return SKSSM_EINVAL;
    const size_t chunk = size_t(unroll) * 4096;
    if (read_bytes == 0 || read_bytes % chunk != 0) return SKSSM_ESHAPE;
    const size_t nchunks = read_bytes / chunk;
    int m = 0;
    if (write_bytes > 0) {
        if (read_bytes % write_bytes != 0) return SKSSM_ESHAPE;
        const size_t ratio = read_bytes / write_bytes;
        if (ratio > size_t(unroll) || unroll % int(ratio) != 0) return SKSSM_ESHAPE;
        m = int(ratio);
    } else if (blocks == 0) {
        return SKSSM_EINVAL;  // a read-only run needs a bounded grid
    }
    const size_t grid = blocks > 0 ? size_t(blocks) : nchunks;
    if (grid > 0x7fffffffu) return SKSSM_ESHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f32x4* s4 = static_cast<const f32x4*>(src);
    f32x4* d4 = static_cast<f32x4*>(dst);
    const bool nt = flags & 1;
    auto go = [&](auto U) {
        constexpr int u = decltype(U)::value;
        if (nt) launch_stream<u, true>(m, grid, s, s4, nchunks, d4);
        else launch_stream<u, false>(m, grid, s, s4, nchunks, d4);
    };
    switch (unroll) {
        case 4: go(std::integral_constant<int, 4>()); break;
        case 8: go(std::integral_constant<int, 8>()); break;
        default: go(std::integral_constant<int, 16>()); break;
    }
    return hipGetLastError() == hipSuccess ? SKSSM_OK : SKSSM_ELAUNCH;
}
