// SketchSSM decode read (sketch heads and dense-fallback heads) for gfx950.
//
// One launch serves one decode step of a layer.  Work items are (b, h) pairs.
// Blocks are laid out along the plan's head order: first one block per item of
// every dense head (a dense item streams its whole fp32 state, ~21x the bytes
// of a rank-6 sketch item), then, per sketch head from high rank buckets to
// low, tiles of 16 batch rows.  Consecutive blocks land on different XCDs, so
// the heavy dense items spread over the whole chip first.
//
// Sketch tile (256 threads, one 16-lane row per item):
//   * the head's coefficient map F (r x K) is staged once in LDS;
//   * the row loads q, k, v, decay (and beta) of the current token and appends
//     them to window slot `pos`;
//   * it sweeps the window back to the last flush: for the current token and
//     then slots pos-1 .. 0, s = k_i . u, intra += beta_i s v_i, u <- M_i^T u,
//     starting at u = q, so that u ends as q~ (page "SketchSSM: Write to the
//     Full State, Read from a Compact Sketch", Abstract: buffered keys and
//     values between state updates);
//   * c_m = F_m . q~ (16-lane DPP reductions) and y = sum_m c_m Z_m + intra
//     (same Abstract: sketch vectors combined with query-dependent
//     coefficients, no full-state read).
// Dense item (256 threads): the state rows are streamed with 16-byte loads
// issued before the sweep; one row sweeps the window; then y = S_0^T q~ + intra
// with a fixed-order LDS reduction over the key dim.
//
// The key dim is 128 = 16 lanes x 8 elements; a lane owns value columns
// 8l .. 8l+7 for l < V/8.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "sketchssm_internal.h"

namespace skssm {

struct ReadArgs {
    const float* S;
    const float* Z;
    const float* frames;
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* beta;
    void* kbuf;
    void* vbuf;
    float* abuf;
    float* bbuf;
    float* y;
    int B, H, pos;
    int n_dense;       // dense heads lead the order
    int tiles;         // ceil(B / 16) tiles per sketch head
    int dense_blocks;  // n_dense * B
};

constexpr int kReadThreads = 256;
constexpr int kRowsPerTile = kReadThreads / 16;

// ---------------------------------------------------------------------------
// The window sweep of one item, run by one 16-lane row (lane l owns key
// elements 8l..8l+7 and, for l < V/8, value elements 8l..8l+7).  Appends the
// current token to slot pos.  Returns u = q~ and the buffered tokens' term.
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
__device__ __forceinline__ void row_sweep(const ReadArgs& A, size_t item, int l, float (&u)[8],
                                          float (&intra)[8]) {
    using V8 = Vec8<QT>;
    constexpr int K = kK;
    constexpr int W = kW;
    constexpr int VL = V / 8;  // lanes that own value columns
    const int pos = A.pos;
    const bool vl = l < VL;

    // current token
    const typename V8::raw_t qr = V8::load(A.q, item * K + 8 * l);
    const typename V8::raw_t kr = V8::load(A.k, item * K + 8 * l);
    typename V8::raw_t vr = V8::zero();
    if (vl) vr = V8::load(A.v, item * V + 8 * l);
    float q[8], kc[8], vc[8];
    V8::unpack(qr, q);
    V8::unpack(kr, kc);
    V8::unpack(vr, vc);
    float ac[8];
    float bc = 1.f;
    if (KIND == SKSSM_KDA) {
        load8f(A.a + item * K + 8 * l, ac);
    } else {
        ac[0] = A.a[item];
    }
    if (KIND != SKSSM_MAMBA2) bc = A.beta[item];

    // append to slot pos
    const size_t slot = item * W + pos;
    V8::store(A.kbuf, slot * K + 8 * l, kr);
    if (vl) V8::store(A.vbuf, slot * V + 8 * l, vr);
    if (KIND == SKSSM_KDA) {
        store8f(A.abuf + slot * K + 8 * l, ac);
    } else if (l == 0) {
        A.abuf[slot] = ac[0];
    }
    if (KIND != SKSSM_MAMBA2 && l == 0) A.bbuf[slot] = bc;

    if (KIND == SKSSM_MAMBA2) {
        // Scalar decay: every buffered token sees q scaled by the decays of the
        // tokens after it, so the dot products k_i . q are independent.
        float g = ac[0];
        const float s_cur = row_sum16(dot8(kc, q));
#pragma unroll
        for (int e = 0; e < 8; ++e) intra[e] = s_cur * vc[e];
        for (int i0 = pos - 1; i0 >= 0; i0 -= 4) {
            typename V8::raw_t kw[4], vw[4];
            float aw[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = i0 - c;
                kw[c] = V8::zero();
                vw[c] = V8::zero();
                aw[c] = 1.f;
                if (i >= 0) {
                    const size_t si = item * W + i;
                    kw[c] = V8::load(A.kbuf, si * K + 8 * l);
                    if (vl) vw[c] = V8::load(A.vbuf, si * V + 8 * l);
                    aw[c] = A.abuf[si];
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float kf[8], vf[8];
                V8::unpack(kw[c], kf);
                V8::unpack(vw[c], vf);
                const float s = row_sum16(dot8(kf, q)) * g;
#pragma unroll
                for (int e = 0; e < 8; ++e) intra[e] = fmaf(s, vf[e], intra[e]);
                g *= aw[c];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = g * q[e];
    } else {
        // Delta rule: u <- M_i^T u is a serial chain through the window.
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = q[e];
        {
            const float s = row_sum16(dot8(kc, u));
            const float bs = bc * s;
#pragma unroll
            for (int e = 0; e < 8; ++e) intra[e] = bs * vc[e];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float al = (KIND == SKSSM_KDA) ? ac[e] : ac[0];
                u[e] = al * fmaf(-bs, kc[e], u[e]);
            }
        }
        for (int i0 = pos - 1; i0 >= 0; i0 -= 4) {
            typename V8::raw_t kw[4], vw[4];
            float aw[4][8];
            float bw[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = i0 - c;
                kw[c] = V8::zero();
                vw[c] = V8::zero();
                bw[c] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) aw[c][e] = 1.f;
                if (i >= 0) {
                    const size_t si = item * W + i;
                    kw[c] = V8::load(A.kbuf, si * K + 8 * l);
                    if (vl) vw[c] = V8::load(A.vbuf, si * V + 8 * l);
                    if (KIND == SKSSM_KDA) {
                        load8f(A.abuf + si * K + 8 * l, aw[c]);
                    } else {
                        aw[c][0] = A.abuf[si];
                    }
                    bw[c] = A.bbuf[si];
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float kf[8], vf[8];
                V8::unpack(kw[c], kf);
                V8::unpack(vw[c], vf);
                const float s = row_sum16(dot8(kf, u));
                const float bs = bw[c] * s;
#pragma unroll
                for (int e = 0; e < 8; ++e) intra[e] = fmaf(bs, vf[e], intra[e]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float al = (KIND == SKSSM_KDA) ? aw[c][e] : aw[c][0];
                    u[e] = al * fmaf(-bs, kf[e], u[e]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dense item: y = S_0^T q~ + intra, whole block on one (b, h).
// Thread t < KG*V4 owns float4 column v4 = t % V4 of key rows kg + KG m.
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
__device__ __forceinline__ void dense_item(const ReadArgs& A, const HeadTable& T, int blk) {
    constexpr int K = kK;
    constexpr int V4 = V / 4;
    constexpr int KG = kReadThreads / V4;
    constexpr int NM = (K + KG - 1) / KG;
    __shared__ float qt_s[K];
    __shared__ float intra_s[V];
    __shared__ float4 part[KG * V4];

    const int tid = threadIdx.x;
    const int p = blk / A.B;
    const int b = blk - p * A.B;
    const int h = T.head[p];
    const size_t item = size_t(b) * A.H + h;
    const int v4 = tid % V4;
    const int kg = tid / V4;
    const bool owner = tid < KG * V4;

    // stream the state rows first; the sweep below overlaps their latency
    const float4* S4 = reinterpret_cast<const float4*>(A.S + item * size_t(K) * V);
    float4 sreg[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int kk = kg + KG * m;
        sreg[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (owner && kk < K) sreg[m] = S4[kk * V4 + v4];
    }

    if (tid < 16) {
        float u[8], intra[8];
        row_sweep<KIND, V, QT>(A, item, tid, u, intra);
        store8f(qt_s + 8 * tid, u);
        if (tid < V / 8) store8f(intra_s + 8 * tid, intra);
    }
    __syncthreads();

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int kk = kg + KG * m;
        if (kk < K) {
            const float qk = qt_s[kk];
            acc.x = fmaf(qk, sreg[m].x, acc.x);
            acc.y = fmaf(qk, sreg[m].y, acc.y);
            acc.z = fmaf(qk, sreg[m].z, acc.z);
            acc.w = fmaf(qk, sreg[m].w, acc.w);
        }
    }
    if (owner) part[kg * V4 + v4] = acc;
    __syncthreads();
    if (tid < V4) {
        float4 s = make_float4(intra_s[4 * tid], intra_s[4 * tid + 1], intra_s[4 * tid + 2],
                               intra_s[4 * tid + 3]);
        float4 t = part[tid];
        for (int g = 1; g < KG; ++g) {
            const float4 x = part[g * V4 + tid];
            t.x += x.x;
            t.y += x.y;
            t.z += x.z;
            t.w += x.w;
        }
        s.x += t.x;
        s.y += t.y;
        s.z += t.z;
        s.w += t.w;
        reinterpret_cast<float4*>(A.y + item * V)[tid] = s;
    }
}

// ---------------------------------------------------------------------------
// Sketch tile: 16 batch rows of one sketch head.
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
__device__ __forceinline__ void sketch_tile(const ReadArgs& A, const HeadTable& T, int sb) {
    constexpr int K = kK;
    constexpr int VL = V / 8;
    extern __shared__ float4 fmap_s4[];  // r x K coefficient map
    const float* fmap_s = reinterpret_cast<const float*>(fmap_s4);

    const int tid = threadIdx.x;
    const int p = A.n_dense + sb / A.tiles;
    const int tile = sb - (sb / A.tiles) * A.tiles;
    const int h = T.head[p];
    const int r = T.rank[p];
    const size_t frow = T.frow[p];
    const size_t zrow = T.zrow[p];

    {
        const float4* src = reinterpret_cast<const float4*>(A.frames + frow * K);
        const int n4 = r * (K / 4);
        for (int e = tid; e < n4; e += kReadThreads) fmap_s4[e] = src[e];
    }

    const int row = tid >> 4;
    const int l = tid & 15;
    const int b = tile * kRowsPerTile + row;
    const bool active = b < A.B;
    const size_t item = size_t(b) * A.H + h;

    float u[8], yacc[8];
    if (active) row_sweep<KIND, V, QT>(A, item, l, u, yacc);
    __syncthreads();
    if (!active) return;

    const float* Zi = A.Z + (zrow * A.B + size_t(b) * r) * V;
    for (int m0 = 0; m0 < r; m0 += 4) {
        float zr[4][8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zr[c][e] = 0.f;
            if (m0 + c < r && l < VL) load8f(Zi + size_t(m0 + c) * V + 8 * l, zr[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (m0 + c < r) {
                float f[8];
                const float* fr = fmap_s + (m0 + c) * K + 8 * l;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = fr[e];
                const float cm = row_sum16(dot8(f, u));
#pragma unroll
                for (int e = 0; e < 8; ++e) yacc[e] = fmaf(cm, zr[c][e], yacc[e]);
            }
        }
    }
    if (l < VL) store8f(A.y + item * V + 8 * l, yacc);
}

template <int KIND, int V, typename QT>
__global__ __launch_bounds__(kReadThreads) void read_kernel(ReadArgs A, HeadTable T) {
    const int blk = blockIdx.x;
    if (blk < A.dense_blocks) {
        dense_item<KIND, V, QT>(A, T, blk);
    } else {
        sketch_tile<KIND, V, QT>(A, T, blk - A.dense_blocks);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
static hipError_t launch_read_t(const ReadArgs& a, const HeadTable& t, int grid, size_t lds,
                                hipStream_t s) {
    hipLaunchKernelGGL((read_kernel<KIND, V, QT>), dim3(grid), dim3(kReadThreads), lds, s, a, t);
    return hipGetLastError();
}

template <int KIND, typename QT>
static hipError_t launch_read_v(int V, const ReadArgs& a, const HeadTable& t, int grid, size_t lds,
                                hipStream_t s) {
    switch (V) {
        case 64: return launch_read_t<KIND, 64, QT>(a, t, grid, lds, s);
        case 80: return launch_read_t<KIND, 80, QT>(a, t, grid, lds, s);
        case 128: return launch_read_t<KIND, 128, QT>(a, t, grid, lds, s);
    }
    return hipErrorInvalidValue;
}

template <typename QT>
static hipError_t launch_read_k(int kind, int V, const ReadArgs& a, const HeadTable& t, int grid,
                                size_t lds, hipStream_t s) {
    switch (kind) {
        case SKSSM_MAMBA2: return launch_read_v<SKSSM_MAMBA2, QT>(V, a, t, grid, lds, s);
        case SKSSM_GDN: return launch_read_v<SKSSM_GDN, QT>(V, a, t, grid, lds, s);
        case SKSSM_KDA: return launch_read_v<SKSSM_KDA, QT>(V, a, t, grid, lds, s);
    }
    return hipErrorInvalidValue;
}

static sketchssm_status run_read(const sketchssm_shape& sh, const HeadTable& t, int n_dense,
                                 int max_rank, const float* S, const float* Z, const float* frames,
                                 const void* q, const void* k, const void* v, const float* a,
                                 const float* beta, void* kbuf, void* vbuf, float* abuf,
                                 float* bbuf, int32_t pos, float* y, void* stream) {
    const bool delta = sh.kind != SKSSM_MAMBA2;
    const int n_sketch = sh.H - n_dense;
    if (!q || !k || !v || !a || !kbuf || !vbuf || !abuf || !y) return SKSSM_EINVAL;
    if (delta != (beta != nullptr) || delta != (bbuf != nullptr)) return SKSSM_EINVAL;
    if (n_dense > 0 && !S) return SKSSM_EINVAL;
    if (n_sketch > 0 && (!Z || !frames)) return SKSSM_EINVAL;
    if (pos < 0 || pos >= sh.W) return SKSSM_EINVAL;
    const void* ptrs[] = {S, Z, frames, q, k, v, a, beta, kbuf, vbuf, abuf, bbuf, y};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return SKSSM_EALIGN;

    ReadArgs A;
    A.S = S;
    A.Z = Z;
    A.frames = frames;
    A.q = q;
    A.k = k;
    A.v = v;
    A.a = a;
    A.beta = beta;
    A.kbuf = kbuf;
    A.vbuf = vbuf;
    A.abuf = abuf;
    A.bbuf = bbuf;
    A.y = y;
    A.B = sh.B;
    A.H = sh.H;
    A.pos = pos;
    A.n_dense = n_dense;
    A.tiles = (sh.B + kRowsPerTile - 1) / kRowsPerTile;
    A.dense_blocks = n_dense * sh.B;
    const long grid = long(A.dense_blocks) + long(n_sketch) * A.tiles;
    if (grid <= 0 || grid > 0x7fffffffL) return SKSSM_ESHAPE;
    const size_t lds = size_t(n_sketch > 0 ? max_rank : 0) * kK * sizeof(float);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = sh.qkv == SKSSM_BF16
                             ? launch_read_k<Bf16Tag>(sh.kind, sh.V, A, t, int(grid), lds, s)
                             : launch_read_k<F32Tag>(sh.kind, sh.V, A, t, int(grid), lds, s);
    return e == hipSuccess ? SKSSM_OK : SKSSM_ELAUNCH;
}

}  // namespace skssm

using namespace skssm;

extern "C" sketchssm_status sketchssm_decode_read(const sketchssm_plan* plan, const float* S,
                                                  const float* Z, const float* frames,
                                                  const void* q, const void* k, const void* v,
                                                  const float* a, const float* beta, void* kbuf,
                                                  void* vbuf, float* abuf, float* bbuf,
                                                  int32_t pos, float* y, void* stream) {
    if (!plan) return SKSSM_EINVAL;
    return run_read(plan->shape, plan->table, plan->n_dense, plan->max_rank, S, Z, frames, q, k,
                    v, a, beta, kbuf, vbuf, abuf, bbuf, pos, y, stream);
}

extern "C" sketchssm_status sketchssm_dense_read(const sketchssm_shape* shape, const float* S,
                                                 const void* q, const void* k, const void* v,
                                                 const float* a, const float* beta, void* kbuf,
                                                 void* vbuf, float* abuf, float* bbuf,
                                                 int32_t pos, float* y, void* stream) {
    const sketchssm_status st = check_shape(shape);
    if (st != SKSSM_OK) return st;
    HeadTable t;
    dense_table(*shape, &t);
    return run_read(*shape, t, shape->H, 0, S, nullptr, nullptr, q, k, v, a, beta, kbuf, vbuf,
                    abuf, bbuf, pos, y, stream);
}
