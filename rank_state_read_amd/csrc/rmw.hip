// Standard per-token decode for gfx950: the full state is read and written for
// every token.  This is the baseline that the SketchSSM pages quote their
// kernel speedups against (page "SketchSSM: Write to the Full State, Read from
// a Compact Sketch", Abstract: speedups over the standard vLLM decode), kept
// here so the same comparison can be made on MI355X.  Per (b, h):
//   S <- M S + beta k v^T,   y = S^T q
// with Mamba-2 M = a I (beta = 1), GDN M = alpha (I - beta k k^T),
// KDA M = (I - beta k k^T) diag(alpha).
//
// One block per item with V/16 waves.  Wave w holds value columns 16w..16w+15
// for all 128 key rows in registers (lane l, register (kt, r) <-> key row
// 16 kt + 4 (l/16) + r, column 16 w + l % 16), loaded with buffer
// instructions.  Both sums over keys (the erase term k^T S and the output
// S^T q) are a per-lane sum over the lane's 32 rows plus two exchanges between
// quarter-waves, so after the token is staged in LDS no barrier is needed
// until the updated state leaves as whole rows staged through LDS.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "sketchssm_internal.h"
#include "state_tiles.h"

namespace skssm {

struct RmwArgs {
    float* S;
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* beta;
    float* y;
    int Hk, share;  // key/query heads; each serves `share` consecutive heads
};

template <typename QT>
__device__ __forceinline__ float rmw_load1(const void* base, size_t elem) {
    if constexpr (std::is_same<QT, Bf16Tag>::value)
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[elem]) << 16);
    else
        return static_cast<const float*>(base)[elem];
}

// Sum over the four lanes l % 16 + 16 j; every lane gets the same bits.
__device__ __forceinline__ float quarter_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// Six waves per SIMD: three 512-thread (V = 128) blocks per CU keep enough of
// the state stream in flight.
template <int KIND, int V, typename QT>
__global__ __launch_bounds__(V / 16 * 64) __attribute__((amdgpu_waves_per_eu(6)))
void rmw_kernel(RmwArgs A) {
    constexpr int K = kK;
    constexpr bool DELTA = KIND != SKSSM_MAMBA2;
    constexpr bool KDA = KIND == SKSSM_KDA;
    __shared__ __align__(16) float qs[K];
    __shared__ __align__(16) float ks[K];
    __shared__ __align__(16) float als[KDA ? K : 4];
    __shared__ __align__(16) float st[2 * 16 * (V + 4)];  // the state on its way out

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int lq = lane >> 4;
    const int v0 = 16 * w;
    const size_t item = blockIdx.x;
    const size_t h = item % (size_t(A.Hk) * A.share);
    const size_t itemk = (item / (size_t(A.Hk) * A.share)) * A.Hk + h / A.share;  // (b, key head)

    // the token: q, k (and KDA decays) to LDS as fp32; this lane's value
    if (tid < K) {
        qs[tid] = rmw_load1<QT>(A.q, itemk * K + tid);
        ks[tid] = rmw_load1<QT>(A.k, itemk * K + tid);
        if (KDA) als[tid] = A.a[item * K + tid];
    }
    const float a_s = KDA ? 1.f : A.a[item];
    const float bt = DELTA ? A.beta[item] : 1.f;
    const float vc = rmw_load1<QT>(A.v, item * V + v0 + lr);

    // the state: this wave's 16 columns, all key rows
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(A.S + item * size_t(K) * V, K * V * 4);
    const int svo = (4 * lq * V + v0 + lr) * 4;
    f32x4 s[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s[kt][rr] = buffer_load_f32(srs, svo, (16 * kt + rr) * V * 4);
    __syncthreads();

    // erase term of this lane's column: GDN k^T S, KDA k^T diag(alpha) S
    float wc = 0.f;
    if (DELTA) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(ks + 16 * kt + 4 * lq);
            f32x4 a4 = {1.f, 1.f, 1.f, 1.f};
            if (KDA) a4 = *reinterpret_cast<const f32x4*>(als + 16 * kt + 4 * lq);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) wc = fmaf(KDA ? k4[rr] * a4[rr] : k4[rr], s[kt][rr], wc);
            if (DELTA) __builtin_amdgcn_sched_barrier(0);
        }
        wc = quarter_sum(wc);
    }

    // S <- M S + beta k v^T, then y = S^T q
    //   Mamba-2  a S + k v
    //   GDN      alpha S + beta k (v - alpha w)
    //   KDA      alpha_row S + beta k (v - w)
    const float vt = KDA ? vc - wc : DELTA ? vc - a_s * wc : vc;
    float yc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(ks + 16 * kt + 4 * lq);
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(qs + 16 * kt + 4 * lq);
        f32x4 a4 = {a_s, a_s, a_s, a_s};
        if (KDA) a4 = *reinterpret_cast<const f32x4*>(als + 16 * kt + 4 * lq);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            s[kt][rr] = fmaf(a4[rr], s[kt][rr], bt * k4[rr] * vt);
            yc = fmaf(q4[rr], s[kt][rr], yc);
        }
        // one tile's operands at a time: keeps the delta-rule instances within their
        // register budget instead of preloading all of them
        if (DELTA) __builtin_amdgcn_sched_barrier(0);
    }
    yc = quarter_sum(yc);
    if (lq == 0) A.y[item * V + v0 + lr] = yc;
    store_state_tiles<V>(s, st, srs, tid);
}

template <int KIND, int V, typename QT>
static hipError_t launch_rmw_t(const RmwArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((rmw_kernel<KIND, V, QT>), dim3(grid), dim3(V / 16 * 64), 0, s, a);
    return hipGetLastError();
}

template <int KIND, typename QT>
static hipError_t launch_rmw_v(int V, const RmwArgs& a, int grid, hipStream_t s) {
    switch (V) {
        case 64: return launch_rmw_t<KIND, 64, QT>(a, grid, s);
        case 80: return launch_rmw_t<KIND, 80, QT>(a, grid, s);
        case 96: return launch_rmw_t<KIND, 96, QT>(a, grid, s);
        case 112: return launch_rmw_t<KIND, 112, QT>(a, grid, s);
        case 128: return launch_rmw_t<KIND, 128, QT>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <typename QT>
static hipError_t launch_rmw_k(int kind, int V, const RmwArgs& a, int grid, hipStream_t s) {
    switch (kind) {
        case SKSSM_MAMBA2: return launch_rmw_v<SKSSM_MAMBA2, QT>(V, a, grid, s);
        case SKSSM_GDN: return launch_rmw_v<SKSSM_GDN, QT>(V, a, grid, s);
        case SKSSM_KDA: return launch_rmw_v<SKSSM_KDA, QT>(V, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace skssm

using namespace skssm;

extern "C" sketchssm_status sketchssm_rmw_step(const sketchssm_shape* shape, float* S,
                                               const void* q, const void* k, const void* v,
                                               const float* a, const float* beta, float* y,
                                               void* stream) {
    const sketchssm_status st = check_shape(shape);
    if (st != SKSSM_OK) return st;
    const bool delta = shape->kind != SKSSM_MAMBA2;
    if (!S || !q || !k || !v || !a || !y) return SKSSM_EINVAL;
    if (delta != (beta != nullptr)) return SKSSM_EINVAL;
    const void* ptrs[] = {S, q, k, v, a, beta, y};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return SKSSM_EALIGN;
    RmwArgs A;
    A.S = S;
    A.q = q;
    A.k = k;
    A.v = v;
    A.a = a;
    A.beta = beta;
    A.y = y;
    A.Hk = kq_heads_of(*shape);
    A.share = shape->H / A.Hk;
    const long grid = long(shape->B) * shape->H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = shape->qkv == SKSSM_BF16
                             ? launch_rmw_k<Bf16Tag>(shape->kind, shape->V, A, int(grid), s)
                             : launch_rmw_k<F32Tag>(shape->kind, shape->V, A, int(grid), s);
    return e == hipSuccess ? SKSSM_OK : SKSSM_ELAUNCH;
}
