// Device helpers shared by the SketchSSM kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sketchssm_internal.h"

namespace skssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Loads of data that a launch reads exactly once and whose every instruction
// covers whole 128-byte lines (window keys and values, the current token's
// q, k, v, a dense item's state).  The non-temporal hint marks the lines as
// streaming; on MI355X a plain stream of whole lines measured ~15% faster with
// it (7.1 against 6.2 TB/s read-only, 6.2 against 5.4 TB/s with one byte
// written per eight read).  Data read in pieces smaller than a line by
// different instructions (scalar decays and betas, sketch rows at a 320-byte
// item stride, a flush's state columns) measured slower with the hint and
// keeps ordinary loads, as do keys shared by several heads, which are reused.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ldnt_u4(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldnt_f4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ldnt_f(const float* p) { return __builtin_nontemporal_load(p); }

// ---------------------------------------------------------------------------
// 8-element vectors of the q/k/v dtype.  A 16-lane row holds one K = 128
// vector as 8 consecutive elements per lane (one 16-byte load for bf16).
// ---------------------------------------------------------------------------
struct Bf16Tag {};
struct F32Tag {};

template <typename QT>
struct Vec8;

template <>
struct Vec8<Bf16Tag> {
    struct raw_t {
        uint4 w;
    };
    static constexpr int kElemBytes = 2;
    __device__ static __forceinline__ raw_t load(const void* base, size_t elem) {
        raw_t r;
        r.w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        return r;
    }
    __device__ static __forceinline__ raw_t load_nt(const void* base, size_t elem) {
        raw_t r;
        r.w = ldnt_u4(static_cast<const uint16_t*>(base) + elem);
        return r;
    }
    // 8 elements at byte offset voff + soff of a buffer resource (streaming or not)
    __device__ static __forceinline__ raw_t load_buf_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff);
    __device__ static __forceinline__ raw_t load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff);
    __device__ static __forceinline__ void store(void* base, size_t elem, const raw_t& r) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = r.w;
    }
    __device__ static __forceinline__ raw_t zero() {
        raw_t r;
        r.w = make_uint4(0u, 0u, 0u, 0u);
        return r;
    }
    __device__ static __forceinline__ void unpack(const raw_t& r, float* f) {
        const uint32_t w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

template <>
struct Vec8<F32Tag> {
    struct raw_t {
        float4 a, b;
    };
    static constexpr int kElemBytes = 4;
    __device__ static __forceinline__ raw_t load(const void* base, size_t elem) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        raw_t r;
        r.a = p[0];
        r.b = p[1];
        return r;
    }
    __device__ static __forceinline__ raw_t load_nt(const void* base, size_t elem) {
        const float* p = static_cast<const float*>(base) + elem;
        raw_t r;
        r.a = ldnt_f4(p);
        r.b = ldnt_f4(p + 4);
        return r;
    }
    __device__ static __forceinline__ raw_t load_buf_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff);
    __device__ static __forceinline__ raw_t load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff);
    __device__ static __forceinline__ void store(void* base, size_t elem, const raw_t& r) {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
        p[0] = r.a;
        p[1] = r.b;
    }
    __device__ static __forceinline__ raw_t zero() {
        raw_t r;
        r.a = make_float4(0.f, 0.f, 0.f, 0.f);
        r.b = r.a;
        return r;
    }
    __device__ static __forceinline__ void unpack(const raw_t& r, float* f) {
        f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
        f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
    }
};

__device__ __forceinline__ void load8f(const float* p, float* f) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void load8f_nt(const float* p, float* f) {
    const float4 a = ldnt_f4(p);
    const float4 b = ldnt_f4(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void store8f(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// ---------------------------------------------------------------------------
// Sum over the 16 lanes of a DPP row.  Butterfly of four DPP adds (swap
// neighbours, swap pairs, mirror half-rows, mirror rows); IEEE addition is
// commutative, so every lane ends with the bitwise same sum.  All 16 lanes of
// the row must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    x += dpp_mov<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
    float s0 = a[0] * b[0];
    float s1 = a[1] * b[1];
    s0 = fmaf(a[2], b[2], s0);
    s1 = fmaf(a[3], b[3], s1);
    s0 = fmaf(a[4], b[4], s0);
    s1 = fmaf(a[5], b[5], s1);
    s0 = fmaf(a[6], b[6], s0);
    s1 = fmaf(a[7], b[7], s1);
    return s0 + s1;
}

// Raw buffer access: one 32-bit per-lane byte offset plus a wave-uniform byte
// offset, so rows far apart cost no per-lane 64-bit address arithmetic.  The
// resource covers `bytes` from `base`; accesses beyond it read 0 / are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                             0x00020000 /* 32-bit data format */);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

__device__ __forceinline__ uint4 buffer_load_u4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming (non-temporal) buffer loads: 16 bytes and 4 bytes.
__device__ __forceinline__ uint4 buffer_load_u4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 2));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float buffer_load_f32_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), 2));
}

__device__ __forceinline__ void buffer_store_f32(float x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, 0);
}

__device__ __forceinline__ Vec8<Bf16Tag>::raw_t Vec8<Bf16Tag>::load_buf_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                                        uint32_t soff) {
    raw_t r;
    r.w = buffer_load_u4_nt(rs, voff, soff);
    return r;
}

__device__ __forceinline__ Vec8<F32Tag>::raw_t Vec8<F32Tag>::load_buf_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                                      uint32_t soff) {
    raw_t r;
    const uint4 a = buffer_load_u4_nt(rs, voff, soff);
    const uint4 b = buffer_load_u4_nt(rs, voff + 16, soff);
    r.a = make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w));
    r.b = make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w));
    return r;
}

__device__ __forceinline__ Vec8<Bf16Tag>::raw_t Vec8<Bf16Tag>::load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                                     uint32_t soff) {
    raw_t r;
    r.w = buffer_load_u4(rs, voff, soff);
    return r;
}

__device__ __forceinline__ Vec8<F32Tag>::raw_t Vec8<F32Tag>::load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                                   uint32_t soff) {
    raw_t r;
    const uint4 a = buffer_load_u4(rs, voff, soff);
    const uint4 b = buffer_load_u4(rs, voff + 16, soff);
    r.a = make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w));
    r.b = make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w));
    return r;
}

// D(16x16) += A(16x4) B(4x16), fp32 in and out.  Operand lanes: A[i][kk] in
// lane i + 16 kk, B[kk][j] in lane j + 16 kk; D[i][j] in lane j + 16 (i / 4),
// register i % 4.
__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace skssm
