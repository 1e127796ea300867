// Writing a block's fp32 state back from the MFMA accumulator layout.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "sketchssm_internal.h"

namespace skssm {

// 16-byte buffer store; NT: non-temporal (streaming) store
template <bool NT = false>
__device__ __forceinline__ void buffer_store_f32x4(f32x4 x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, soff, NT ? 2 : 0);
}

// Store the K x V state held by V / 16 waves (wave w, lane l, tile kt,
// register r <-> S[16 kt + 4 (l / 16) + r][16 w + l % 16]) to its row-major
// place covered by `srs`.  In that layout one store instruction writes four
// 64-byte pieces of four rows; on a stream of states read and written back
// such stores ran ~15% slower than stores of whole rows.  So the state goes
// through LDS TR rows at a time and leaves as contiguous 16-byte stores (the
// block has 4 V threads: TR / 16 stores per thread and round).  NBUF = 2
// alternates two staging areas (one barrier per round), NBUF = 1 reuses one
// (two).  `st` is NBUF x TR x (V + 4) floats of LDS that no wave reads any
// more; the call begins with a barrier, after which they are overwritten.
// NT: the rows leave as non-temporal stores (nothing reads them back soon).
template <int V, int TR = 16, int NBUF = 2, bool NT = false>
__device__ __forceinline__ void store_state_tiles(const f32x4 (&s)[8], float* st, __amdgpu_buffer_rsrc_t srs,
                                                  int tid) {
    static_assert(TR % 16 == 0 && kK % TR == 0 && (NBUF == 1 || NBUF == 2), "tile rows");
    constexpr int VS = V + 4;  // 4 (mod 16) floats: the four quarter-waves' rows start 16 banks apart
    constexpr int NR = kK / TR;
    constexpr int TT = TR / 16;  // 16-row tiles per round
    const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int row = tid / (V / 4), c4 = tid - row * (V / 4);
    __syncthreads();
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
        // with two areas a round's area is rewritten two rounds later, after
        // every thread has passed the barrier that follows its reads
        float* t = st + (rd % NBUF) * TR * VS;
        if (NBUF == 1 && rd > 0) __syncthreads();
#pragma unroll
        for (int j = 0; j < TT; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) t[(16 * j + 4 * lq + rr) * VS + 16 * w + lr] = s[TT * rd + j][rr];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(t + (16 * j + row) * VS + 4 * c4);
            buffer_store_f32x4<NT>(v, srs, (row * V + 4 * c4) * 4, (TR * rd + 16 * j) * V * 4);
        }
    }
}

}  // namespace skssm
