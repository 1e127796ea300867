// SketchSSM decode read (sketch heads and dense-fallback heads) for gfx950.
//
// One launch serves one decode step of a layer; work items are (b, h) pairs.
// Blocks follow the plan's order of the sketch heads, from high rank buckets to
// low, each as blocks of 16 batch rows with one 16-lane DPP row per item; one
// block per item of every dense head comes last.  A dense item streams its
// whole fp32 state (~21x the bytes of a rank-6 sketch item), but its block moves
// fewer bytes than a 16-row sketch block and ends sooner, and a launch usually
// holds more waves than the chip keeps resident (9152 against 8192 for a
// 128-head Nano-shaped layer at batch 256), so the
// blocks that start late, when the first ones end, are best the shortest: the
// longest-first order by block, not by item.
//
// Per item the read
//   * appends the current token (k, v, decay, beta) to window slot `pos`;
//   * sweeps the window back to the last flush: for the current token and then
//     slots pos-1 .. 0, s = k_i . u, intra += beta_i s v_i, u <- M_i^T u,
//     starting at u = q, so that u ends as q~ (page "SketchSSM: Write to the
//     Full State, Read from a Compact Sketch", Abstract: keys and values are
//     held back between state updates);
//   * sketch head: c_m = F_m . q~ and y = sum_m c_m Z_m + intra (same
//     Abstract: the stored sketch rows are mixed with weights taken from the
//     query, S is not touched); dense head: y = S_0^T q~ + intra.
//
// The read is bound by HBM traffic; what costs time is how the bytes are laid
// out, not arithmetic.  The window is slot-major ([W][H][B]), so a block's
// append is one contiguous slab and older slots are read as contiguous runs;
// the sketch is head-major, so a block reads one contiguous span of Z.  Waves
// stay at <= 64 VGPRs (Mamba-2, bf16) so eight are resident per SIMD and the
// per-item round trips overlap across the 128 items each CU owns.
//
// A second instance of the kernel (continuous batching) takes one window
// position per batch row instead of one per launch; a row whose position is
// outside 0 .. W-1 is left idle.
#include <hip/hip_runtime.h>

#include <type_traits>

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
    const int32_t* pos_seq;  // per-sequence window positions (continuous batching) or null
    int B, H, pos;
    int Hk, share;     // key/query heads; each serves `share` consecutive heads
    int n_dense;       // dense heads lead the head table (their blocks run last)
    int tiles;         // ceil(B / 16) blocks per sketch head
    int dense_blocks;  // n_dense * B
};

constexpr int kReadThreads = 256;

// ---------------------------------------------------------------------------
// The item sweep in row layout (one 16-lane row per item; lane l owns key
// elements 8l .. 8l+7 and, for l < V/8, value elements 8l .. 8l+7).  The
// window is walked from the current token back to slot 0 in chunks of CH
// slots.  The kernel keeps each wave small (<= 64 VGPRs) so that eight waves
// per SIMD are resident: with all of a CU's items in flight at once, the
// serial round trips of one item hide behind the others.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
    typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2;
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x),
                                              __builtin_bit_cast(bf16x2, b.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), s, false);
    return s;
}

// k . q for two raw 8-vectors of the q/k/v dtype (bf16: packed dot products)
template <typename QT>
__device__ __forceinline__ float raw_dot8(const typename Vec8<QT>::raw_t& a, const typename Vec8<QT>::raw_t& b) {
    if constexpr (std::is_same<QT, Bf16Tag>::value) {
        return dot8_bf16(a.w, b.w);
    } else {
        float x[8], y[8];
        Vec8<QT>::unpack(a, x);
        Vec8<QT>::unpack(b, y);
        return dot8(x, y);
    }
}

// UPOS: the window position is the same for every row of a wave (a lockstep
// launch, or a dense item's block); a slot's byte offset is then wave-uniform.
template <int KIND, int V, typename QT, bool DEEP = false, bool UPOS = true>
struct RowSweep {
    static constexpr bool KDA = KIND == SKSSM_KDA;
    static constexpr bool DELTA = KIND != SKSSM_MAMBA2;
    // window slots per round trip: the bf16 GDN instances have registers to
    // spare (a 96-VGPR budget), so with DEEP they fetch four slots at a time
    static constexpr int CH =
        KDA ? 1 : (DEEP && KIND == SKSSM_GDN && std::is_same<QT, Bf16Tag>::value) ? 4 : 2;
    static constexpr int NA = KDA ? 8 : 1;  // decay values per slot and lane
    using V8 = Vec8<QT>;

    // Per-item LDS staging of the current token, written when it is first
    // read and copied to window slot pos after the item's output: the token
    // is neither held in registers through the sweep nor read from HBM twice.
    static constexpr int E = V8::kElemBytes;
    static constexpr int kStageK = 0;                        // raw key, K elements
    static constexpr int kStageV = kStageK + kK * E;         // raw value, V elements
    static constexpr int kStageA = kStageV + V * E;          // KDA: K decays (fp32)
    static constexpr int kStageS = kStageA + (KDA ? kK * 4 : 0);  // scalar decay, beta
    static constexpr int kStageBytes = kStageS + 16;

    // Appends the current token to window slot pos from the staging copy.
    // Called after the item's loads have been consumed: stores count in the
    // same in-order memory counter as loads, so a store issued ahead of a load
    // would make the wait for that load also wait for the store.
    __device__ __forceinline__ static void append(const ReadArgs& A, int b, int h, int l, int pos,
                                                  const char* stg) {
        const float* ss = reinterpret_cast<const float*>(stg + kStageS);
        const typename V8::raw_t kc = V8::load(stg + kStageK, 8 * l);
        typename V8::raw_t vc = V8::zero();
        if (l < V / 8) vc = V8::load(stg + kStageV, 8 * l);
        const size_t slot = (size_t(pos) * A.H + h) * A.B + b;
        // a shared key slot is written once, by the first head of its group
        if (h % A.share == 0) {
            const size_t kslot = (size_t(pos) * A.Hk + h / A.share) * A.B + b;
            V8::store(A.kbuf, kslot * kK + 8 * l, kc);
        }
        if (l < V / 8) V8::store(A.vbuf, slot * V + 8 * l, vc);
        if (KDA) {
            float ac[8];
            load8f(reinterpret_cast<const float*>(stg + kStageA) + 8 * l, ac);
            store8f(A.abuf + slot * kK + 8 * l, ac);
        } else if (l == 0) {
            A.abuf[slot] = ss[0];
        }
        if (DELTA && l == 0) A.bbuf[slot] = ss[1];
    }

    // Sweeps the window of `item` and stages the current token in `stg`.
    // Mamba-2: u = q~ is returned as (gtot, qr) with q~ = gtot q; delta: u = q~.
    __device__ __forceinline__ static void run(const ReadArgs& A, int b, int h, int l, int pos,
                                               typename V8::raw_t& qr, float (&u)[8],
                                               float (&acc)[8], float& gtot, char* stg) {
        const size_t item = size_t(b) * A.H + h;
        const int kh = h / A.share;                  // key/query head
        const size_t itemk = size_t(b) * A.Hk + kh;
        const bool vl = l < V / 8;
        // lanes >= V/8 own no value elements; they re-read lane 0's chunk (in
        // bounds, never stored) so that no load sits in a divergent branch,
        // which would make the compiler wait for it at the branch's end
        const int vo = vl ? 8 * l : 0;
        // The window arrays as buffer resources: a slot adds a fixed byte
        // stride, the item and lane a per-lane byte offset (one register per
        // array for every slot).  Each array is below 2^31 bytes for every
        // shape the plan accepts.
        const uint32_t kstride = uint32_t(A.Hk) * uint32_t(A.B) * (kK * E);
        const uint32_t vstride = uint32_t(A.H) * uint32_t(A.B) * (V * E);
        const uint32_t astride = uint32_t(A.H) * uint32_t(A.B) * (NA == 8 ? kK * 4 : 4);
        const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(A.kbuf, kW * kstride);
        const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(A.vbuf, kW * vstride);
        const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(A.abuf, kW * astride);
        const uint32_t bstride = uint32_t(A.H) * uint32_t(A.B) * 4;
        const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(A.bbuf, DELTA ? kW * bstride : 0);
        const uint32_t ko = uint32_t((size_t(kh) * A.B + b) * kK + 8 * l) * E;
        const uint32_t vo_b = uint32_t((size_t(h) * A.B + b) * V + vo) * E;
        const uint32_t hb = uint32_t(size_t(h) * A.B + b);
        const uint32_t ao = KDA ? (hb * kK + 8 * l) * 4 : hb * 4;
        typename V8::raw_t kw[CH], vw[CH];
        float aw[CH][NA], bw[CH];
        // every slot of a chunk is loaded (a slot before the window's start
        // re-reads slot 0) and the ones past the start are then masked: the
        // loads stay free of branches
        auto load_chunk = [&](int i0) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const uint32_t ic = uint32_t(i0 - j >= 0 ? i0 - j : 0);
                // a uniform slot offset goes in the scalar offset (read from
                // the first lane, so that it stays in a scalar register even
                // where the compiler computes it with a vector instruction),
                // else in the lane's
                auto off = [&](uint32_t lane, uint32_t stride, uint32_t& v) {
                    v = UPOS ? lane : lane + ic * stride;
                    return UPOS ? uint32_t(__builtin_amdgcn_readfirstlane(int(ic * stride))) : 0u;
                };
                uint32_t vk, vv, va, vb;
                const uint32_t sk = off(ko, kstride, vk), sv = off(vo_b, vstride, vv);
                const uint32_t sa = off(ao, astride, va), sb = off(hb * 4, bstride, vb);
                if (A.share > 1) kw[j] = V8::load_buf(krs, vk, sk);
                else kw[j] = V8::load_buf_nt(krs, vk, sk);
                vw[j] = V8::load_buf_nt(vrs, vv, sv);
                if (KDA) {
                    const uint4 a0 = buffer_load_u4_nt(ars, va, sa);
                    const uint4 a1 = buffer_load_u4_nt(ars, va + 16, sa);
                    const uint32_t aa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                    for (int e = 0; e < NA; ++e) aw[j][e] = __uint_as_float(aa[e]);
                } else {
                    aw[j][0] = buffer_load_f32(ars, int(va), int(sa));
                }
                bw[j] = DELTA ? buffer_load_f32(brs, int(vb), int(sb)) : 0.f;
            }
        };

        // q and k are streamed unless several heads share them (then reused)
        typename V8::raw_t kc;
        if (A.share > 1) {
            qr = V8::load(A.q, itemk * kK + 8 * l);
            kc = V8::load(A.k, itemk * kK + 8 * l);
        } else {
            qr = V8::load_nt(A.q, itemk * kK + 8 * l);
            kc = V8::load_nt(A.k, itemk * kK + 8 * l);
        }
        const typename V8::raw_t vc = V8::load_nt(A.v, item * V + vo);
        float ac[NA];
        if (KDA) load8f_nt(A.a + item * kK + 8 * l, ac);
        else ac[0] = A.a[item];
        const float bc = DELTA ? A.beta[item] : 1.f;
        // keep the token's loads together: the staging stores below must not
        // pull a wait in between them
        __builtin_amdgcn_sched_barrier(0);
        V8::store(stg + kStageK, 8 * l, kc);
        if (vl) V8::store(stg + kStageV, 8 * l, vc);
        if (KDA) store8f(reinterpret_cast<float*>(stg + kStageA) + 8 * l, ac);
        if (l == 0) {
            float* ss = reinterpret_cast<float*>(stg + kStageS);
            ss[0] = ac[0];
            ss[1] = bc;
        }

        float g = 1.f;
        if (!DELTA) {
            float vf[8];
            V8::unpack(vc, vf);
            const float s = row_sum16(raw_dot8<QT>(kc, qr));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = s * vf[e];
            g = ac[0];
        } else {
            V8::unpack(qr, u);
            float kf[8], vf[8];
            V8::unpack(kc, kf);
            V8::unpack(vc, vf);
            const float bs = bc * row_sum16(dot8(kf, u));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[e] = bs * vf[e];
                u[e] = (KDA ? ac[e] : ac[0]) * fmaf(-bs, kf[e], u[e]);
            }
        }

        for (int i0 = pos - 1; i0 >= 0; i0 -= CH) {
            load_chunk(i0);
#pragma unroll
            for (int j = 1; j < CH; ++j) {
                if (i0 - j < 0) {
                    kw[j] = V8::zero();
                    vw[j] = V8::zero();
#pragma unroll
                    for (int e = 0; e < NA; ++e) aw[j][e] = 1.f;
                    bw[j] = 0.f;
                }
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                float vf[8];
                V8::unpack(vw[j], vf);
                if (!DELTA) {
                    const float s = row_sum16(raw_dot8<QT>(kw[j], qr)) * g;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(s, vf[e], acc[e]);
                    g *= aw[j][0];
                } else {
                    float kf[8];
                    V8::unpack(kw[j], kf);
                    const float bs = bw[j] * row_sum16(dot8(kf, u));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        acc[e] = fmaf(bs, vf[e], acc[e]);
                        u[e] = (KDA ? aw[j][e] : aw[j][0]) * fmaf(-bs, kf[e], u[e]);
                    }
                }
            }
        }
        gtot = g;
    }
};

// ---------------------------------------------------------------------------
// Sketch block: kRows consecutive batch rows of one sketch head.
// ---------------------------------------------------------------------------
constexpr int kRows = kReadThreads / 16;
constexpr int kMapRows = 16;  // coefficient-map rows staged in LDS at a time
static_assert(kK == 128, "the map granule order is laid out for 32 granules per row");

template <int KIND, int V, typename QT, bool SEQ>
__device__ __forceinline__ void sketch_block(const ReadArgs& A, const HeadTable& T, int sb,
                                             float4* lds4) {
    constexpr int K = kK;
    constexpr int VL = V / 8;
    constexpr bool M2 = KIND == SKSSM_MAMBA2;
    using V8 = Vec8<QT>;
    using RS = RowSweep<KIND, V, QT, !SEQ, !SEQ>;
    // LDS: kRows token staging rows, then the coefficient map
    constexpr int kMapOff4 = kRows * RS::kStageBytes / 16;
    char* stg = reinterpret_cast<char*>(lds4) + (threadIdx.x >> 4) * RS::kStageBytes;
    const float* fmap_s = reinterpret_cast<const float*>(lds4 + kMapOff4);

    const int tid = threadIdx.x;
    const int row = tid >> 4;
    const int l = tid & 15;
    const int tile = sb / A.tiles;
    const int p = A.n_dense + tile;
    const int bt = sb - tile * A.tiles;
    const int h = T.head[p];
    const int r = T.rank[p];
    const size_t frow = T.frow[p];
    const size_t zrow = T.zrow[p];
    const int b = bt * kRows + row;
    // window position of this row's sequence; rows outside the batch, or whose
    // position is outside 0 .. W-1, do nothing
    const int pos = SEQ ? (b < A.B ? A.pos_seq[b] : -1) : A.pos;
    const bool active = b < A.B && pos >= 0 && pos < kW;
    const size_t item = size_t(b) * A.H + h;
    const float* Zi = A.Z + (zrow * A.B + size_t(b) * r) * V;

    // the coefficient map straight into LDS, kMapRows rows at a time (wave w
    // fills 1 KB pieces w, w+4, ...); most heads need a single piece, and the
    // block's LDS stays small enough for eight resident blocks per CU.  Inside
    // a map row the 16-byte granules are stored as 0, 2, .., 30, 1, 3, .., 31:
    // lane l reads its key elements 8l .. 8l+7 as granules l and 16 + l, so
    // each of its two reads covers 256 contiguous bytes across the 16 lanes
    // (every bank once).  A piece with an odd row count also fills the slots
    // of one row more (the launcher sizes the map for an even row count).
    auto stage_map = [&](int m0) {
        const float4* fsrc = reinterpret_cast<const float4*>(A.frames + (frow + m0) * K);
        const int n4 = min(kMapRows, r - m0) * (K / 4);
        const int w = tid >> 6, L = tid & 63;
        for (int c = w; c * 64 < n4; c += kReadThreads / 64) {
            const int d = c * 64 + L;  // the LDS granule this lane fills
            const int sl = d & (K / 4 - 1);
            const int g = (d & ~(K / 4 - 1)) | (sl < K / 8 ? 2 * sl : 2 * (sl - K / 8) + 1);
            const int e = min(g, n4 - 1);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(fsrc + e),
                                             (__attribute__((address_space(3))) void*)(lds4 + kMapOff4 + c * 64),
                                             16, 0, 0);
        }
    };
    stage_map(0);

    // y = sum_m (F_m . q~) Z_m + intra, ZR sketch rows per round trip (four
    // for the lockstep bf16 GDN instances, which have the registers, else two)
    constexpr int ZR = (!SEQ && KIND == SKSSM_GDN && std::is_same<QT, Bf16Tag>::value) ? 4 : 2;
    float z[ZR][8];
    auto load_z = [&](int m, int mend) {
#pragma unroll
        for (int j = 0; j < ZR; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) z[j][e] = 0.f;
        if (l < VL) {
#pragma unroll
            for (int j = 0; j < ZR; ++j)
                if (m + j < mend) load8f(Zi + size_t(m + j) * V + 8 * l, z[j]);
        }
    };

    typename V8::raw_t qr;
    float u[8], acc[8], gtot = 1.f;
    if (SEQ) {
        // rows of one tile may sit at different window positions: wait for the
        // map first, so that no barrier after the sweeps holds every wave to
        // the tile's longest window
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the map has landed
        __syncthreads();
        if (active) RS::run(A, b, h, l, pos, qr, u, acc, gtot, stg);
    } else {
        // the map arrives while the sweep runs
        if (active) RS::run(A, b, h, l, pos, qr, u, acc, gtot, stg);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the map has landed
        __syncthreads();
    }
    if (M2) {
        float q[8];
        V8::unpack(qr, q);
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = gtot * q[e];
    }

    for (int m0 = 0; m0 < r; m0 += kMapRows) {
        if (m0 > 0) {
            __syncthreads();  // every row is done with the previous piece
            stage_map(m0);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
        const int mend = min(r, m0 + kMapRows);
        if (!active) continue;
        for (int m = m0; m < mend; m += ZR) {
            load_z(m, mend);
#pragma unroll
            for (int j = 0; j < ZR; ++j) {
                if (m + j < mend) {
                    float f[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = fmap_s[(m + j - m0) * K + 4 * l + e];
                        f[4 + e] = fmap_s[(m + j - m0) * K + K / 2 + 4 * l + e];
                    }
                    const float cj = row_sum16(dot8(f, u));
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(cj, z[j][e], acc[e]);
                }
            }
        }
    }
    if (!active) return;
    if (l < VL) store8f(A.y + item * V + 8 * l, acc);
    RS::append(A, b, h, l, pos, stg);
}

// ---------------------------------------------------------------------------
// Dense block: y = S_0^T q~ + intra for one (b, h).  Row 0 sweeps the window
// while the block streams the state with 16-byte loads, PH rows per thread
// per round trip; thread t < KG*V4 owns float4 column t % V4 of key rows
// t / V4 + KG m, summed over the key rows in a fixed order through LDS.
// ---------------------------------------------------------------------------
template <int V>
struct DenseLds {
    static constexpr int V4 = V / 4;
    static constexpr int KG = kReadThreads / V4;
    static constexpr size_t bytes = size_t(kK + V) * 4 + size_t(KG) * V4 * 16;
    // Mamba-2, lockstep: each row's window term (score, decay, value) after the
    // token staging
    static constexpr size_t spread_bytes = size_t(2 * 16 + 16 * V) * 4;
};

template <int KIND, int V, typename QT, bool SEQ>
__device__ __forceinline__ void dense_block(const ReadArgs& A, const HeadTable& T, int blk,
                                            float4* lds4) {
    constexpr int K = kK;
    constexpr int V4 = V / 4;
    constexpr int KG = kReadThreads / V4;
    constexpr int NM = (K + KG - 1) / KG;
    constexpr int PH = 4;
    constexpr bool M2 = KIND == SKSSM_MAMBA2;
    using V8 = Vec8<QT>;
    float4* part = lds4;                                          // [KG * V4]
    float* qt_s = reinterpret_cast<float*>(lds4 + KG * V4);       // [K]
    float* intra_s = qt_s + K;                                    // [V]

    const int tid = threadIdx.x;
    const int p = blk / A.B;
    const int b = blk - p * A.B;
    const int h = T.head[p];
    const size_t item = size_t(b) * A.H + h;
    int pos = A.pos;
    if (SEQ) {
        pos = __builtin_amdgcn_readfirstlane(A.pos_seq[b]);
        if (pos < 0 || pos >= kW) return;  // the whole block: this sequence is idle
    }
    const int v4 = tid % V4;
    const int kg = tid / V4;
    const bool owner = tid < KG * V4;
    const float4* S4 = reinterpret_cast<const float4*>(A.S + item * size_t(K) * V);

    float4 sreg[PH];
#pragma unroll
    for (int j = 0; j < PH; ++j) {
        const int kk = kg + KG * j;
        sreg[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (owner && kk < K) sreg[j] = ldnt_f4(reinterpret_cast<const float*>(S4 + kk * V4 + v4));
    }
    using RS = RowSweep<KIND, V, QT, !SEQ>;
    char* stg = reinterpret_cast<char*>(lds4) + DenseLds<V>::bytes;
    if constexpr (M2 && !SEQ) {
        // Mamba-2 decays are scalars, so the window's terms do not depend on
        // one another: row j > 0 reads window slot pos - j and forms its k . q
        // while row 0 reads the current token, all in one round trip; row 0
        // then adds the terms in the row sweep's order (slot pos - 1 first, the
        // same decay products), which gives the sweep's result bit for bit.
        float* sc_s = reinterpret_cast<float*>(stg + RS::kStageBytes);  // [16] raw scores
        float* a_s = sc_s + 16;                                          // [16] decays
        float* v_s = a_s + 16;                                           // [16][V] values
        const int row = tid >> 4, l = tid & 15;
        const int kh = h / A.share;
        const size_t itemk = size_t(b) * A.Hk + kh;
        const bool vl = l < V / 8;
        const int vo = vl ? 8 * l : 0;
        // rows past the window's start re-read the current token (in bounds,
        // unused), so the loads need no branch
        const bool win = row > 0 && row <= pos;
        const size_t i = size_t(win ? pos - row : 0);
        const size_t kslot = (i * A.Hk + kh) * A.B + b;
        const size_t slot = (i * A.H + h) * A.B + b;
        const typename V8::raw_t qj = V8::load(A.q, itemk * kK + 8 * l);
        const typename V8::raw_t kw = V8::load(win ? A.kbuf : A.k, (win ? kslot : itemk) * kK + 8 * l);
        const typename V8::raw_t vw = V8::load(win ? A.vbuf : A.v, (win ? slot : item) * V + vo);
        const float aw = (win ? A.abuf + slot : A.a + item)[0];
        const float sj = row_sum16(raw_dot8<QT>(kw, qj));
        float vf[8];
        V8::unpack(vw, vf);
        if (row == 0) {
            V8::store(stg + RS::kStageK, 8 * l, kw);
            if (vl) V8::store(stg + RS::kStageV, 8 * l, vw);
            if (l == 0) reinterpret_cast<float*>(stg + RS::kStageS)[0] = aw;
        } else if (win) {
            if (vl) store8f(v_s + row * V + vo, vf);
            if (l == 0) {
                sc_s[row] = sj;
                a_s[row] = aw;
            }
        }
        __syncthreads();
        if (row == 0) {
            float acc[8], u[8], q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = sj * vf[e];
            float g = aw;
            for (int j = 1; j <= pos; ++j) {
                const float s = sc_s[j] * g;
                float vv[8];
                load8f(v_s + j * V + vo, vv);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(s, vv[e], acc[e]);
                g *= a_s[j];
            }
            V8::unpack(qj, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = g * q[e];
            store8f(qt_s + 8 * l, u);
            if (vl) store8f(intra_s + 8 * l, acc);
            RS::append(A, b, h, l, pos, stg);
        }
    } else if (tid < 16) {
        typename V8::raw_t qr;
        float u[8], acc[8], g = 1.f;
        RS::run(A, b, h, tid, pos, qr, u, acc, g, stg);
        if (M2) {
            float q[8];
            V8::unpack(qr, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = g * q[e];
        }
        store8f(qt_s + 8 * tid, u);
        if (tid < V / 8) store8f(intra_s + 8 * tid, acc);
        RS::append(A, b, h, tid, pos, stg);
    }
    __syncthreads();

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int m0 = 0; m0 < NM; m0 += PH) {
        if (m0 > 0) {
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                const int kk = kg + KG * (m0 + j);
                sreg[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (owner && kk < K) sreg[j] = ldnt_f4(reinterpret_cast<const float*>(S4 + kk * V4 + v4));
            }
        }
#pragma unroll
        for (int j = 0; j < PH; ++j) {
            const int kk = kg + KG * (m0 + j);
            if (kk < K) {
                const float qk = qt_s[kk];
                acc.x = fmaf(qk, sreg[j].x, acc.x);
                acc.y = fmaf(qk, sreg[j].y, acc.y);
                acc.z = fmaf(qk, sreg[j].z, acc.z);
                acc.w = fmaf(qk, sreg[j].w, acc.w);
            }
        }
    }
    if (owner) part[kg * V4 + v4] = acc;
    __syncthreads();
    if (tid < V4) {
        float4 t = part[tid];
        for (int g = 1; g < KG; ++g) {
            const float4 x = part[g * V4 + tid];
            t.x += x.x;
            t.y += x.y;
            t.z += x.z;
            t.w += x.w;
        }
        const float4 s = make_float4(intra_s[4 * tid] + t.x, intra_s[4 * tid + 1] + t.y,
                                     intra_s[4 * tid + 2] + t.z, intra_s[4 * tid + 3] + t.w);
        reinterpret_cast<float4*>(A.y + item * V)[tid] = s;
    }
}

// Waves per SIMD the register budget is sized for: 8 (64 VGPRs) where the
// sweep fits (Mamba-2 with bf16 tokens up to V = 112), 5 (96 VGPRs) for the
// wider per-channel / fp32 variants, 4 (128) for the fp32 V = 128 per-sequence
// instances, which need a little more.
template <int KIND, int V, typename QT, bool SEQ>
struct ReadOccupancy {
    static constexpr bool kF32 = std::is_same<QT, F32Tag>::value;
    static constexpr int value = (KIND == SKSSM_MAMBA2 && V <= 112 && !kF32) ? 8
                                 : (SEQ && kF32 && V == 128)               ? 4
                                                                            : 5;
};

// SEQ: every sequence has its own window position (continuous batching);
// otherwise the whole batch is at position A.pos.
template <int KIND, int V, typename QT, bool SEQ>
__global__ __launch_bounds__(kReadThreads)
__attribute__((amdgpu_waves_per_eu(ReadOccupancy<KIND, V, QT, SEQ>::value)))
void read_kernel(ReadArgs A, HeadTable T) {
    extern __shared__ float4 lds4[];  // token staging + coefficient map (sketch) or reduction buffers (dense)
    // sketch tiles first, the dense heads' items last
    const int blk = blockIdx.x;
    const int sketch_blocks = int(gridDim.x) - A.dense_blocks;
    if (blk < sketch_blocks) {
        sketch_block<KIND, V, QT, SEQ>(A, T, blk, lds4);
    } else {
        dense_block<KIND, V, QT, SEQ>(A, T, blk - sketch_blocks, lds4);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT>
static hipError_t launch_read_t(const ReadArgs& a, const HeadTable& t, int grid, size_t lds,
                                hipStream_t s) {
    if (a.pos_seq)
        hipLaunchKernelGGL((read_kernel<KIND, V, QT, true>), dim3(grid), dim3(kReadThreads), lds, s, a, t);
    else
        hipLaunchKernelGGL((read_kernel<KIND, V, QT, false>), dim3(grid), dim3(kReadThreads), lds, s, a, t);
    return hipGetLastError();
}

template <int KIND, typename QT>
static hipError_t launch_read_v(int V, const ReadArgs& a, const HeadTable& t, int grid, size_t lds,
                                hipStream_t s) {
    switch (V) {
        case 64: return launch_read_t<KIND, 64, QT>(a, t, grid, lds, s);
        case 80: return launch_read_t<KIND, 80, QT>(a, t, grid, lds, s);
        case 96: return launch_read_t<KIND, 96, QT>(a, t, grid, lds, s);
        case 112: return launch_read_t<KIND, 112, QT>(a, t, grid, lds, s);
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
                                 float* bbuf, int32_t pos, const int32_t* pos_seq, float* y,
                                 void* stream) {
    const bool delta = sh.kind != SKSSM_MAMBA2;
    const int n_sketch = sh.H - n_dense;
    if (!q || !k || !v || !a || !kbuf || !vbuf || !abuf || !y) return SKSSM_EINVAL;
    if (delta != (beta != nullptr) || delta != (bbuf != nullptr)) return SKSSM_EINVAL;
    if (n_dense > 0 && !S) return SKSSM_EINVAL;
    if (n_sketch > 0 && (!Z || !frames)) return SKSSM_EINVAL;
    if (!pos_seq && (pos < 0 || pos >= sh.W)) return SKSSM_EINVAL;
    if (reinterpret_cast<uintptr_t>(pos_seq) & 3u) return SKSSM_EALIGN;
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
    A.pos_seq = pos_seq;
    A.Hk = kq_heads_of(sh);
    A.share = sh.H / A.Hk;
    A.n_dense = n_dense;
    A.tiles = (sh.B + kRows - 1) / kRows;
    A.dense_blocks = n_dense * sh.B;
    const long grid = long(A.dense_blocks) + long(n_sketch) * A.tiles;
    if (grid <= 0 || grid > 0x7fffffffL) return SKSSM_ESHAPE;
    // per-item token staging (must match RowSweep's layout)
    const size_t eb = sh.qkv == SKSSM_BF16 ? 2 : 4;
    const size_t stage = kK * eb + size_t(sh.V) * eb + (sh.kind == SKSSM_KDA ? kK * 4 : 0) + 16;
    size_t lds = 0;
    // the map piece: min(max_rank, kMapRows) rows, rounded up to even (the
    // staging fills whole 64-granule chunks)
    const int map_rows = ((max_rank < kMapRows ? max_rank : kMapRows) + 1) & ~1;
    if (n_sketch > 0) lds = kRows * stage + size_t(map_rows) * kK * sizeof(float);
    if (n_dense > 0) {
        size_t dl = stage;
        const bool spread = sh.kind == SKSSM_MAMBA2 && !pos_seq;  // the dense block's window terms
        switch (sh.V) {
            case 64: dl += DenseLds<64>::bytes + (spread ? DenseLds<64>::spread_bytes : 0); break;
            case 80: dl += DenseLds<80>::bytes + (spread ? DenseLds<80>::spread_bytes : 0); break;
            case 96: dl += DenseLds<96>::bytes + (spread ? DenseLds<96>::spread_bytes : 0); break;
            case 112: dl += DenseLds<112>::bytes + (spread ? DenseLds<112>::spread_bytes : 0); break;
            default: dl += DenseLds<128>::bytes + (spread ? DenseLds<128>::spread_bytes : 0); break;
        }
        lds = lds > dl ? lds : dl;
    }
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
                    v, a, beta, kbuf, vbuf, abuf, bbuf, pos, nullptr, y, stream);
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
                    abuf, bbuf, pos, nullptr, y, stream);
}

extern "C" sketchssm_status sketchssm_decode_read_seq(const sketchssm_plan* plan, const float* S,
                                                      const float* Z, const float* frames,
                                                      const void* q, const void* k, const void* v,
                                                      const float* a, const float* beta, void* kbuf,
                                                      void* vbuf, float* abuf, float* bbuf,
                                                      const int32_t* pos, float* y, void* stream) {
    if (!plan || !pos) return SKSSM_EINVAL;
    return run_read(plan->shape, plan->table, plan->n_dense, plan->max_rank, S, Z, frames, q, k,
                    v, a, beta, kbuf, vbuf, abuf, bbuf, 0, pos, y, stream);
}
