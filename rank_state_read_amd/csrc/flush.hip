// SketchSSM flush + sketch for gfx950.
//
// One block per (b, h) item; consecutive blocks walk the batch of one head, so
// the head's basis rows stay in L2.  The block has V/16 waves; wave w owns
// value columns 16w .. 16w+15 of the item's fp32 state and holds all K = 128
// key rows of them in registers as eight 16x16 MFMA accumulator tiles
// (lane l, register r <-> S[16 kt + 4 (l/16) + r][16 w + l%16]).  In one pass
// over the state it
//   1. applies the window's n held-back tokens (page "SketchSSM: Write to the
//      Full State, Read from a Compact Sketch", Abstract: keys and values wait
//      for a periodic exact update; W = 16 on the Nemotron Nano 9B v2
//      calibration card, "Contents"), and
//   2. emits the sketch Z = Omega_r S of the updated state for a sketch head
//      (same Abstract: the update is the one time S is read, and the basis
//      directions' outputs are kept from it).
//
// The n updates are applied in chunked ("WY") form, with slots 0..n-1,
// gamma_i = prod_{m<=i} alpha_m and sigma_i = prod_{m>i} alpha_m (per channel
// for KDA, scalars otherwise; slots >= n act as alpha = 1, k = v = 0, beta = 0):
//   Mamba-2:  S_n = gamma S_0 + sum_i (sigma_i k_i) v_i^T
//   delta:    G = (gamma_i * k_i)^T S_0 rows (W x V),
//             L_il = beta_i sum_c k_i[c] k_l[c] prod_{l<m<=i} alpha_m[c]  (l < i),
//             (I + L) U = diag(beta) (V_w - G),
//             S_n = gamma * S_0 + sum_i (sigma_i * k_i) u_i^T.
// The state tiles serve directly as the B operand of G and Z: the register
// index r of a tile is used as the 4-wide K step, which only permutes the
// order of the key sum, and the A operand is read with the same permutation.
//
// Latency: the small loads (window, decays, basis rows) are issued before the
// 40-64 KB state load, so staging them never waits behind the state; scalar
// decay products are formed per thread from the 16 decays, so Mamba-2 needs a
// single barrier per item.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "sketchssm_internal.h"

namespace skssm {

struct FlushArgs {
    float* S;
    float* Z;
    const float* basis;
    const void* kbuf;
    const void* vbuf;
    const float* abuf;
    const float* bbuf;
    int B, H, n_tokens, basis_rows;
    int omt;  // 16-row tiles of the largest rank (the Omega^T stride is 16 omt + 4)
};

// LDS row strides chosen so that the MFMA operand reads of a half-wave hit
// distinct banks: rows read by lanes 16 apart differ by 16 banks.
constexpr int kKtStride = kK + 16;  // [i][k]
constexpr int kKgStride = 20;       // [k][i]
template <int V>
struct VStride {
    static constexpr int value = (V % 32 == 16) ? V : V + 16;
};

template <int KIND, int V>
struct FlushLds {
    static constexpr bool delta = KIND != SKSSM_MAMBA2;
    static constexpr bool kda = KIND == SKSSM_KDA;
    static constexpr int US = VStride<V>::value;
    static constexpr int kt = 0;                                  // [16][kKtStride]
    static constexpr int u = kt + 16 * kKtStride;                 // [16][US]
    static constexpr int nd = kda ? 16 * kK : 0;                  // KDA decay arrays
    static constexpr int alpha = u + 16 * US;
    static constexpr int gam = alpha + nd;
    static constexpr int sig = gam + nd;
    static constexpr int kr = sig + nd;                           // delta: raw k [16][K]
    static constexpr int kg = kr + (delta ? 16 * kK : 0);         // delta: [K][kKgStride]
    static constexpr int lm = kg + (delta ? kK * kKgStride : 0);  // delta: L [16][16]
    static constexpr int om = lm + (delta ? 256 : 0);             // Omega^T [K][16 omt + 4]
    static size_t bytes(int omt) { return size_t(om + (omt > 0 ? kK * (16 * omt + 4) : 0)) * 4; }
};

template <int KIND, int V, typename QT>
__global__ __launch_bounds__(V / 16 * 64) void flush_kernel(FlushArgs A, HeadTable T) {
    using V8 = Vec8<QT>;
    using L = FlushLds<KIND, V>;
    constexpr int K = kK;
    constexpr int W = kW;
    constexpr int NW = V / 16;
    constexpr int NT = NW * 64;
    constexpr bool DELTA = L::delta;
    constexpr bool KDA = L::kda;
    constexpr int US = L::US;
    constexpr int KCH = W * K / 8;  // 8-element key chunks of the window
    constexpr int VCH = W * V / 8;  // 8-element value chunks
    constexpr int ACH = W * K / 4;  // float4 chunks of KDA decays
    constexpr int NA = (ACH + NT - 1) / NT;
    extern __shared__ float4 lds4[];
    float* sm = reinterpret_cast<float*>(lds4);
    float* Kt = sm + L::kt;
    float* U = sm + L::u;
    float* al = sm + L::alpha;
    float* gam = sm + L::gam;
    float* sig = sm + L::sig;
    float* Kr = sm + L::kr;
    float* KgT = sm + L::kg;
    float* Lm = sm + L::lm;
    float* OmT = sm + L::om;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;  // column inside the wave's 16
    const int lq = lane >> 4;  // 4-row group
    const int p = blockIdx.x / A.B;
    const int b = blockIdx.x - p * A.B;
    const int h = T.head[p];
    const int r = T.rank[p];
    const int g = T.group[p];
    const size_t item = size_t(b) * A.H + h;
    const int n = A.n_tokens;
    const bool sketch = r > 0 && A.Z != nullptr;
    const int oms = 16 * A.omt + 4;
    const int v0 = 16 * w;
    // window slot i of this item: [W][H][B] layout, slot-major
    auto wslot = [&](int i) { return (size_t(i) * A.H + h) * A.B + b; };

    // ---- 1. small loads first: window chunk, decays, betas ----
    typename V8::raw_t kraw = V8::zero(), vraw = V8::zero();
    const int ki = tid >> 4, kk0 = (tid & 15) * 8;            // key chunk of this thread
    const int vi = tid / (V / 8), vc0 = (tid % (V / 8)) * 8;  // value chunk of this thread
    float4 a4[KDA ? NA : 1];
    float as[W], bs[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        as[i] = 1.f;
        bs[i] = 0.f;
    }
    if (n > 0) {
        if (tid < KCH && ki < n) kraw = V8::load(A.kbuf, wslot(ki) * K + kk0);
        if (tid < VCH && vi < n) vraw = V8::load(A.vbuf, wslot(vi) * V + vc0);
        if (KDA) {
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int c = tid + j * NT;
                a4[j] = make_float4(1.f, 1.f, 1.f, 1.f);
                if (c < ACH && (c >> 5) < n)
                    a4[j] = *reinterpret_cast<const float4*>(A.abuf + wslot(c >> 5) * K + (c & 31) * 4);
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) as[i] = i < n ? A.abuf[wslot(i)] : 1.f;
        }
        if (DELTA) {
#pragma unroll
            for (int i = 0; i < W; ++i) bs[i] = i < n ? A.bbuf[wslot(i)] : 0.f;
        }
    }

    // ---- 2. the state: this wave's 16 columns, all key rows ----
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(A.S + item * size_t(K) * V, K * V * 4);
    const int svo = (4 * lq * V + v0 + lr) * 4;  // this lane's byte offset in a 16-row tile
    f32x4 s[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s[kt][rr] = buffer_load_f32(srs, svo, (16 * kt + rr) * V * 4);

    // ---- 3. stage operands ----
    if (sketch) {
        // basis rows, transposed; consecutive threads write consecutive LDS words
        const float* om = A.basis + size_t(g) * A.basis_rows * K;
        const int orows = 16 * ((r + 15) / 16);
        for (int e = tid; e < orows * K; e += NT) {
            const int kk = e / orows, m = e - kk * orows;
            OmT[kk * oms + m] = m < r ? om[m * K + kk] : 0.f;
        }
    }
    float gamW = 1.f;
    if (n > 0) {
        if (KDA) {
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int c = tid + j * NT;
                if (c < ACH) reinterpret_cast<float4*>(al)[c] = a4[j];
            }
            __syncthreads();
            for (int c = tid; c < K; c += NT) {
                float pr = 1.f;
                for (int i = 0; i < W; ++i) {
                    pr *= al[i * K + c];
                    gam[i * K + c] = pr;
                }
                float sf = 1.f;
                for (int i = W - 1; i >= 0; --i) {
                    sig[i * K + c] = sf;
                    sf *= al[i * K + c];
                }
            }
            __syncthreads();
        }
        // prefix / suffix decay products of this thread's key slot (scalar kinds)
        float gi = 1.f, si = 1.f;
        if (!KDA) {
#pragma unroll
            for (int i = 0; i < W; ++i) {
                gamW *= as[i];
                if (i <= ki) gi *= as[i];
                if (i > ki) si *= as[i];
            }
        }
        if (tid < KCH) {
            float f[8];
            V8::unpack(kraw, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = kk0 + e;
                const float sg = KDA ? sig[ki * K + kk] : si;
                Kt[ki * kKtStride + kk] = f[e] * sg;
                if (DELTA) {
                    const float gm = KDA ? gam[ki * K + kk] : gi;
                    Kr[ki * K + kk] = f[e];
                    KgT[kk * kKgStride + ki] = f[e] * gm;
                }
            }
        }
        if (tid < VCH) {
            float f[8];
            V8::unpack(vraw, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) U[vi * US + vc0 + e] = f[e];
        }
    }
    __syncthreads();

    if (n > 0) {
        if (DELTA) {
            // 4a. L: row i of 16 lanes handles token i against every earlier token
            {
                const int i = tid >> 4;
                const int l16 = tid & 15;
                if (i >= 1 && i < W) {
                    float kv[8], R[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        kv[e] = Kr[i * K + 8 * l16 + e];
                        R[e] = 1.f;
                    }
                    float bi = 0.f;
#pragma unroll
                    for (int ii = 0; ii < W; ++ii)
                        if (ii == i) bi = bs[ii];
                    for (int j = i - 1; j >= 0; --j) {
                        float aj = 1.f;
                        if (!KDA) {
#pragma unroll
                            for (int ii = 0; ii < W; ++ii)
                                if (ii == j + 1) aj = as[ii];
                        }
                        float t = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            R[e] *= KDA ? al[(j + 1) * K + 8 * l16 + e] : aj;
                            t = fmaf(kv[e] * R[e], Kr[j * K + 8 * l16 + e], t);
                        }
                        const float sum = row_sum16(t);
                        if (l16 == 0) Lm[i * 16 + j] = bi * sum;
                    }
                }
            }
            // 4b. G tile for this wave's columns: rows = tokens, K summed in registers
            f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int ss = 0; ss < 4; ++ss)
                    gacc = mfma_16x16x4(KgT[(16 * kt + 4 * lq + ss) * kKgStride + lr], s[kt][ss], gacc);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                float bsel = 0.f;
#pragma unroll
                for (int ii = 0; ii < W; ++ii)
                    if (ii == 4 * lq + rr) bsel = bs[ii];
                float* up = U + (4 * lq + rr) * US + v0 + lr;
                *up = bsel * (*up - gacc[rr]);
            }
            __syncthreads();
            // 4c. forward substitution (I + L) U = rhs, one lane per column
            if (lane < 16) {
                const int col = v0 + lane;
                float uc[W];
#pragma unroll
                for (int ii = 0; ii < W; ++ii) {
                    float acc = U[ii * US + col];
#pragma unroll
                    for (int jj = 0; jj < ii; ++jj) acc = fmaf(-Lm[ii * 16 + jj], uc[jj], acc);
                    uc[ii] = acc;
                }
#pragma unroll
                for (int ii = 0; ii < W; ++ii) U[ii * US + col] = uc[ii];
            }
            __syncthreads();
        }

        // 5. S <- gamma * S + Kt^T U, stored back
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            f32x4 acc;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float gw = KDA ? gam[(W - 1) * K + 16 * kt + 4 * lq + rr] : gamW;
                acc[rr] = gw * s[kt][rr];
            }
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) {
                const int ii = 4 * ss + lq;
                acc = mfma_16x16x4(Kt[ii * kKtStride + 16 * kt + lr], U[ii * US + v0 + lr], acc);
            }
            s[kt] = acc;
        }
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) buffer_store_f32(s[kt][rr], srs, svo, (16 * kt + rr) * V * 4);
    }

    // 6. Z = Omega_r S for a sketch head
    if (sketch) {
        float* Zi = A.Z + (size_t(T.zrow[p]) * A.B + size_t(b) * r) * V;
        const int mts = (r + 15) / 16;
        for (int mt = 0; mt < mts; ++mt) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int ss = 0; ss < 4; ++ss)
                    z = mfma_16x16x4(OmT[(16 * kt + 4 * lq + ss) * oms + 16 * mt + lr], s[kt][ss], z);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = 16 * mt + 4 * lq + rr;
                if (m < r) Zi[size_t(m) * V + v0 + lr] = z[rr];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
static hipError_t launch_flush_t(const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    const size_t lds = FlushLds<KIND, V>::bytes(a.omt);
    auto fn = flush_kernel<KIND, V, QT>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(V / 16 * 64), lds, s, a, t);
    return hipGetLastError();
}

template <int KIND, typename QT>
static hipError_t launch_flush_v(int V, const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    switch (V) {
        case 64: return launch_flush_t<KIND, 64, QT>(a, t, grid, s);
        case 80: return launch_flush_t<KIND, 80, QT>(a, t, grid, s);
        case 128: return launch_flush_t<KIND, 128, QT>(a, t, grid, s);
    }
    return hipErrorInvalidValue;
}

template <typename QT>
static hipError_t launch_flush_k(int kind, int V, const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    switch (kind) {
        case SKSSM_MAMBA2: return launch_flush_v<SKSSM_MAMBA2, QT>(V, a, t, grid, s);
        case SKSSM_GDN: return launch_flush_v<SKSSM_GDN, QT>(V, a, t, grid, s);
        case SKSSM_KDA: return launch_flush_v<SKSSM_KDA, QT>(V, a, t, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace skssm

using namespace skssm;

extern "C" sketchssm_status sketchssm_flush(const sketchssm_plan* plan, float* S, float* Z,
                                            const float* basis, const void* kbuf,
                                            const void* vbuf, const float* abuf,
                                            const float* bbuf, int32_t n_tokens, void* stream) {
    if (!plan) return SKSSM_EINVAL;
    const sketchssm_shape& sh = plan->shape;
    const bool delta = sh.kind != SKSSM_MAMBA2;
    const int n_sketch = sh.H - plan->n_dense;
    if (!S) return SKSSM_EINVAL;
    if (n_tokens < 0 || n_tokens > sh.W) return SKSSM_EINVAL;
    if (n_sketch > 0 && (!Z || !basis)) return SKSSM_EINVAL;
    if (n_tokens > 0 && (!kbuf || !vbuf || !abuf)) return SKSSM_EINVAL;
    if (n_tokens > 0 && delta && !bbuf) return SKSSM_EINVAL;
    if (!delta && bbuf) return SKSSM_EINVAL;
    const void* ptrs[] = {S, Z, basis, kbuf, vbuf, abuf, bbuf};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return SKSSM_EALIGN;
    if (n_sketch == 0 && n_tokens == 0) return SKSSM_OK;  // nothing to write

    FlushArgs A;
    A.S = S;
    A.Z = n_sketch > 0 ? Z : nullptr;
    A.basis = basis;
    A.kbuf = kbuf;
    A.vbuf = vbuf;
    A.abuf = abuf;
    A.bbuf = bbuf;
    A.B = sh.B;
    A.H = sh.H;
    A.n_tokens = n_tokens;
    A.basis_rows = sh.basis_rows;
    A.omt = n_sketch > 0 ? (plan->max_rank + 15) / 16 : 0;
    const long grid = long(sh.B) * sh.H;
    if (grid > 0x7fffffffL) return SKSSM_ESHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = sh.qkv == SKSSM_BF16
                             ? launch_flush_k<Bf16Tag>(sh.kind, sh.V, A, plan->table, int(grid), s)
                             : launch_flush_k<F32Tag>(sh.kind, sh.V, A, plan->table, int(grid), s);
    return e == hipSuccess ? SKSSM_OK : SKSSM_ELAUNCH;
}
