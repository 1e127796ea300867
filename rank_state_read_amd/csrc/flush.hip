// SketchSSM flush + sketch for gfx950.
//
// One block per (b, h) item; consecutive blocks walk the batch of one head, so
// the head's basis rows stay in L2.  With a row list (continuous batching)
// the blocks walk the listed rows instead, each with its own token count.  The
// block has V/16 waves; wave w owns value columns 16w .. 16w+15 of the item's
// fp32 state and holds all K = 128 key rows of them in registers as eight
// 16x16 MFMA accumulator tiles (lane l, register r <-> S[16 kt + 4 (l/16) + r]
// [16 w + l%16]).  In one pass over the state it
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
//   Mamba-2:  S_n = gamma_W S_0 + sum_i (sigma_i k_i) v_i^T
//   delta:    L_il = beta_i sum_c k_i[c] k_l[c] prod_{l<m<=i} alpha_m[c]  (l < i),
//             T = (I + L)^{-1} diag(beta),
//             U = T V_w - (T (gamma K)) S_0       (the rows u_i, W x V),
//             S_n = gamma_W * S_0 + sum_i (sigma_i * k_i) u_i^T.
// Everything except the two products with S_0 depends on the window alone, so
// it is formed while the state is still on its way from HBM: L, T, the 16 x K
// operand -(T (gamma K)) and the 16 x V tile T V_w.  Once the state has landed
// each wave only runs MFMAs on its own columns -- U (kept in registers, where
// its accumulator layout is already the B operand of the update), the update,
// Z -- with no barrier unless the head's rank exceeds 16 (each further 16-row
// basis tile is staged between two barriers).  The Mamba-2 kernels then store
// the sketch rows and the state as whole rows staged through LDS; the
// delta-rule ones store them from the accumulator layout.
//
// The state tiles serve directly as the B operand of the products with S: the
// register index r of a tile is used as the 4-wide K step, which only permutes
// the order of the key sum, and the A operand is read with the same
// permutation.  Window tokens enter every 16-deep product in the order
// 4 (l/16) + step, so one 16 x 16 accumulator (token rows 4 (l/16) + r) feeds
// the next product without leaving its lane.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "sketchssm_internal.h"
#include "state_tiles.h"

namespace skssm {

struct FlushArgs {
    float* S;
    float* Z;
    const float* basis;
    const void* kbuf;
    const void* vbuf;
    const float* abuf;
    const float* bbuf;
    const int32_t* seqs;  // batch rows to flush (continuous batching) or null: every row
    const int32_t* ntok;  // tokens held back per listed row
    int B, H, n_tokens, basis_rows;
    int Hk, share;  // key heads; each serves `share` consecutive heads
    int nb;   // blocks per head: B, or the number of listed rows
    int omt;  // basis tiles held in LDS: 1 when the plan has sketch heads, else 0
    // the fused last read: the token at window position W-1 (not appended; it is
    // the window's last slot), the coefficient maps and the output
    const void* tq;
    const void* tk;
    const void* tv;
    const float* ta;
    const float* tb;
    const float* frames;
    float* y;
};

// LDS map, in floats.  Row strides are 4 (mod 16) floats: the rows 4 (l/16) + s
// that the four quarter-waves read then start 16 banks apart.
template <int KIND, int V, bool FUSED = false>
struct FlushLds {
    static constexpr bool delta = KIND != SKSSM_MAMBA2;
    static constexpr bool kda = KIND == SKSSM_KDA;
    static constexpr int KS = kK + 4;                      // rows of K floats
    static constexpr int VS = V + 4;                       // rows of V floats
    static constexpr int kt = 0;                           // sigma-scaled keys [16][KS]
    static constexpr int ap = kt + 16 * KS;                // delta: raw keys, then -T(gamma K) [16][KS]
    static constexpr int gw = ap + (delta ? 16 * KS : 0);  // KDA: gamma_W per channel [K]
    static constexpr int vw = gw + (kda ? kK : 0);         // window values [16][VS]
    static constexpr int kg = vw + 16 * VS;                // delta: gamma-scaled keys [16][KS]
    static constexpr int lt = kg + (delta ? 16 * KS : 0);  // delta: L [16][16] (row-major)
    static constexpr int tm = lt + (delta ? 256 : 0);      // delta: T [16][16]
    static constexpr int al = tm + (delta ? 256 : 0);      // KDA: decays [16][K]
    static constexpr int om = al + (kda ? 16 * kK : 0);    // one tile of basis rows [16][K], swizzled
    // fused last read: the query, q~ (delta), (sigma K) q, T^T (sigma K) q, c = F q~,
    // and one 16-row tile of the coefficient map
    static constexpr int qs = om + 16 * kK;
    static constexpr int qt = qs + (FUSED ? kK : 0);
    static constexpr int ws = qt + (FUSED && delta ? kK : 0);
    static constexpr int ts = ws + (FUSED ? 16 : 0);
    static constexpr int cs = ts + (FUSED ? 16 : 0);
    static constexpr int fm = cs + (FUSED ? 16 : 0);
    static size_t bytes(int omt) {
        return FUSED ? size_t(fm + 16 * kK) * 4 : size_t(om + 16 * omt * kK) * 4;
    }
};

// Sum over the four lanes l % 16 + 16 j; every lane gets the same bits.
__device__ __forceinline__ float quarter_sum4(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// One column of the unit lower-triangular solve (I + L) x = b held by a DPP
// row, lane i holding x_i and its row of L: step M broadcasts x_M (final by
// then) from lane M of the row and subtracts L[i][M] x_M in the lanes i > M.
template <int M, int N>
struct TriSolveStep {
    __device__ __forceinline__ static void run(float& x, const float (&lrow)[16], int l16) {
        if constexpr (M < N) {
            const float xm = __int_as_float(
                __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + M, 0xF, 0xF, false));  // row_newbcast:M
            const float nx = fmaf(-lrow[M], xm, x);
            x = l16 > M ? nx : x;
            TriSolveStep<M + 1, N>::run(x, lrow, l16);
        }
    }
};

// Row-local shift toward lane 0 by S lanes (lane j takes lane j + S of its
// DPP row; the last S lanes of the row take `fill`), and toward lane 15.
template <int S>
__device__ __forceinline__ float row_shl(float x, float fill) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x100 + S, 0xF, 0xF, false));
}
template <int S>
__device__ __forceinline__ float row_shr(float x, float fill) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x110 + S, 0xF, 0xF, false));
}

// Occupancy the register budget is sized for: three 512-thread blocks of the
// V = 128 kernels per CU, four of the 320-thread V = 80 ones.
constexpr int kFlushWavesPerEu = 6;

// FUSED: the read of the window's last token and the flush of the full window
// in one pass (see sketchssm_decode_read_flush); the fused KDA instances take
// a 96-VGPR budget, the others fit the plain flush's 80.
template <int KIND, int V, typename QT, bool FUSED>
__global__ __launch_bounds__(V / 16 * 64)
__attribute__((amdgpu_waves_per_eu((FUSED && KIND == SKSSM_KDA) ? 5 : kFlushWavesPerEu)))
void flush_kernel(FlushArgs A, HeadTable T) {
    using V8 = Vec8<QT>;
    using L = FlushLds<KIND, V, FUSED>;
    constexpr int K = kK;
    constexpr int W = kW;
    constexpr int NW = V / 16;
    constexpr bool DELTA = L::delta;
    constexpr bool KDA = L::kda;
    constexpr int KS = L::KS;
    constexpr int VS = L::VS;
    constexpr int VCH = W * V / 8;  // 8-element value chunks of the window
    extern __shared__ float4 lds4[];
    float* sm = reinterpret_cast<float*>(lds4);
    float* Kt = sm + L::kt;
    float* Ap = sm + L::ap;
    float* Gw = sm + L::gw;
    float* Vw = sm + L::vw;
    float* Kg = sm + L::kg;
    float* Lr = sm + L::lt;
    float* Tm = sm + L::tm;
    float* Al = sm + L::al;
    float* Om = sm + L::om;
    float* Qs = sm + L::qs;  // fused: the query
    float* Qt = sm + L::qt;  // fused, delta rule: q~
    float* Ws = sm + L::ws;  // fused, delta rule: (sigma K) q
    float* Ts = sm + L::ts;  // fused, delta rule: T^T (sigma K) q
    float* Cs = sm + L::cs;  // fused: c = F q~ of the current map tile
    float* Fm = sm + L::fm;  // fused: one 16-row tile of the coefficient map

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;  // column inside the wave's 16 / row of an A operand
    const int lq = lane >> 4;  // quarter-wave: 4-row group
    const int p = blockIdx.x / A.nb;
    const int j = blockIdx.x - p * A.nb;
    // batch row and held-back tokens of this block; a listed row outside the
    // batch or a count outside 0 .. W leaves the block idle
    int b = j, n = A.n_tokens;
    if (A.seqs) {
        b = __builtin_amdgcn_readfirstlane(A.seqs[j]);
        n = __builtin_amdgcn_readfirstlane(A.ntok[j]);
        if (b < 0 || b >= A.B || n < 0 || n > W) return;
    }
    const int h = __builtin_amdgcn_readfirstlane(T.head[p]);
    const int r = __builtin_amdgcn_readfirstlane(T.rank[p]);
    const int g = __builtin_amdgcn_readfirstlane(T.group[p]);
    const size_t item = size_t(b) * A.H + h;
    const bool sketch = r > 0 && A.Z != nullptr;
    // no tokens and no sketch to emit (a dense head's initial sketch): the
    // state stays as it is and the block has nothing to read
    if (n == 0 && !sketch) return;
    const int v0 = 16 * w;
    // window slot i of this item: [W][H][B] layout, slot-major (keys: [W][Hk][B])
    auto wslot = [&](int i) { return (size_t(i) * A.H + h) * A.B + b; };
    auto wslotk = [&](int i) { return (size_t(i) * A.Hk + h / A.share) * A.B + b; };

    // fused: coefficient-map rows 16 mt .. 16 mt + 15 into Fm (natural order;
    // rows from r up repeat row r - 1 and are never used)
    auto stage_fmap = [&](int mt) {
        const float* fsrc = A.frames + size_t(T.frow[p]) * K;
        const int wq = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
        for (int jf = 0; jf < (8 + NW - 1) / NW; ++jf) {
            const int qd = wq + jf * NW;  // 64-granule chunk: tile rows 2 qd, 2 qd + 1
            if (qd < 8) {
                const int gi = 64 * qd + lane;
                const int row = 16 * mt + (gi >> 5);
                const int srow = row < r ? row : r - 1;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(fsrc + size_t(srow) * K + 4 * (gi & 31)),
                    (__attribute__((address_space(3))) void*)(Fm + 256 * qd), 16, 0, 0);
            }
        }
    };

    // The state is requested after the window (below), except in the fused
    // Mamba-2 pass, whose window-phase work (the last token's read) is short:
    // there it goes first and that work waits for it (641 against 649 us at a
    // Nano-shaped layer; for the other instances this order measured the same
    // or slower).
    constexpr bool SFIRST = FUSED && KIND == SKSSM_MAMBA2;
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(A.S + item * size_t(K) * V, K * V * 4);
    const int svo = (4 * lq * V + v0 + lr) * 4;  // this lane's byte offset in a 16-row tile
    f32x4 s[8];
    auto load_state = [&]() {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) s[kt][rr] = buffer_load_f32(srs, svo, (16 * kt + rr) * V * 4);
    };
    if (SFIRST) load_state();

    // ---- 1. window loads into registers, issued first ----
    // Every slot is fetched (the window always holds W slots) and slots >= n
    // are masked where the values are used: the loads then need no branches,
    // which would make them wait before the state load is issued.  Lane l of
    // every wave fetches slot l % 16's scalar decay and beta; threads below
    // KCH / VCH fetch one 8-element chunk of the window's keys / values, and
    // for KDA threads fetch 4-channel chunks of the decays.
    constexpr int KCH = W * K / 8;
    constexpr int ACH = W * K / 4;
    constexpr int NT = NW * 64;
    constexpr int NA = KDA ? (ACH + NT - 1) / NT : 1;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    float as_l = 1.f, bs_l = 0.f;
    typename V8::raw_t kraw = V8::zero(), vraw = V8::zero();
    float4 a4[NA];
    const int ki = tid >> 4, kc0 = (tid & 15) * 8;            // key chunk of this thread
    const int vi = tid / (V / 8), vc0 = (tid % (V / 8)) * 8;  // value chunk of this thread
    const size_t itemk = size_t(b) * A.Hk + h / A.share;  // (b, key head)
    if (n > 0) {
        // fused: slot W-1 is the current token, read from its inputs (the
        // source address is selected, so the loads stay outside branches)
        const bool cur_s = FUSED && (lane & 15) == W - 1;
        if (!KDA) as_l = cur_s ? A.ta[item] : A.abuf[wslot(lane & 15)];
        if (DELTA) bs_l = cur_s ? A.tb[item] : A.bbuf[wslot(lane & 15)];
        if (tid < KCH) {
            const bool cur = FUSED && ki == W - 1;
            kraw = V8::load(cur ? A.tk : A.kbuf, cur ? itemk * K + kc0 : wslotk(ki) * K + kc0);
        }
        if (tid < VCH) {
            const bool cur = FUSED && vi == W - 1;
            vraw = V8::load(cur ? A.tv : A.vbuf, cur ? item * V + vc0 : wslot(vi) * V + vc0);
        }
        if (KDA) {
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int c = tid + j * NT;
                const bool cur = FUSED && (c >> 5) == W - 1;
                const float* src = cur ? A.ta + item * K : A.abuf + wslot(c >> 5) * K;
                if (c < ACH) a4[j] = *reinterpret_cast<const float4*>(src + (c & 31) * 4);
            }
        }
    }
    // fused: the query (16 threads, 8 elements each), the first 16 sketch rows
    // of the old sketch for this lane's column (rows lq + 4 j) and the first
    // 16 rows of the coefficient map (straight into LDS)
    typename V8::raw_t qraw = V8::zero();
    float zo[4] = {0.f, 0.f, 0.f, 0.f};
    const float* Zold = sketch ? A.Z + (size_t(T.zrow[p]) * A.B + size_t(b) * r) * V : nullptr;
    if (FUSED) {
        if (tid < K / 8) qraw = V8::load(A.tq, itemk * K + 8 * tid);
        if (sketch) {
#pragma unroll
            for (int jz = 0; jz < 4; ++jz) {
                const int m = min(lq + 4 * jz, r - 1);  // rows >= r are loaded but not used
                zo[jz] = Zold[size_t(m) * V + v0 + lr];
            }
            stage_fmap(0);
        }
    }

    // ---- 2. basis rows, straight into LDS, one 16-row tile at a time (16-byte
    // granules; granule c of row m is stored at slot c ^ (m % 16) so that the
    // sixteen rows one A-operand read touches fall in distinct banks).  Rows
    // from r up to the next multiple of 16 repeat row r - 1: they only feed
    // sketch rows that are never stored.  Holding one tile instead of the
    // largest rank's rows keeps the block's LDS small enough that registers,
    // not LDS, bound the resident blocks (a V = 80 Mamba-2 layer whose largest
    // rank is 49: four 320-thread blocks per CU instead of three).  The first
    // tile is requested here, with the window.
    auto stage_basis = [&](int mt) {
        const float* om = A.basis + size_t(g) * A.basis_rows * K;
#pragma unroll
        for (int j = 0; j < (8 + NW - 1) / NW; ++j) {
            const int qd = wu + j * NW;  // 64-granule chunk: tile rows 2 qd, 2 qd + 1
            if (qd < 8) {
                const int gi = 64 * qd + lane;
                const int m = gi >> 5;
                const int c4 = (gi & 31) ^ m;
                const int row = 16 * mt + m;
                const int srow = row < r ? row : r - 1;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(om + size_t(srow) * K + 4 * c4),
                    (__attribute__((address_space(3))) void*)(Om + 256 * qd), 16, 0, 0);
            }
        }
    };
    if (sketch) stage_basis(0);

    // Window and basis rows first, the state after: while direct-to-LDS loads
    // are outstanding the memory counter cannot tell loads apart, so every
    // later wait would wait for the whole state too.  Waiting here for the
    // small loads (L2 / last-level cache hits) leaves only state loads in
    // flight during the window-only work below, and the MFMAs on the state
    // then wait for each load on its own.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- 3. the state: this wave's 16 columns, all key rows ----
    if (!SFIRST) load_state();

    // ---- 4. window-only work while the state is in flight ----
    // slots >= n act as alpha = 1, beta = 0, k = v = 0
    if (SFIRST) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the state landed with the window
    // (lane l of every DPP row holds slot l's scalar decay and beta)
    as_l = (lane & 15) < n ? as_l : 1.f;
    bs_l = (lane & 15) < n ? bs_l : 0.f;
    float gamW = 1.f;
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
    float zc = 0.f;     // fused: sum_m c_m Z_old[m][column], this lane's column
    float intra = 0.f;  // fused: the buffered tokens' term of the last read, same column
    if (n > 0) {
        if (FUSED && tid < K / 8) {
            float f[8];
            V8::unpack(qraw, f);
            store8f(Qs + 8 * tid, f);
        }
        if (tid < VCH) {
            float f[8];
            V8::unpack(vraw, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = vi < n ? f[e] : 0.f;
            store8f(Vw + vi * VS + vc0, f);
        }
        if (KDA) {
            // raw keys and decays to LDS; channel c's prefix / suffix products
            // are then formed by thread c
            if (tid < KCH) {
                float f[8];
                V8::unpack(kraw, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = ki < n ? f[e] : 0.f;
                store8f(Ap + ki * KS + kc0, f);
            }
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int c = tid + j * NT;
                if (c < ACH) {
                    const bool live = (c >> 5) < n;
                    const float4 v4 = live ? a4[j] : make_float4(1.f, 1.f, 1.f, 1.f);
                    *reinterpret_cast<float4*>(Al + (c >> 5) * K + (c & 31) * 4) = v4;
                }
            }
            __syncthreads();
            if (tid < K) {
                const int c = tid;
                float gm = 1.f;
#pragma unroll 4
                for (int i = 0; i < W; ++i) {
                    gm *= Al[i * K + c];
                    Kg[i * KS + c] = Ap[i * KS + c] * gm;
                }
                Gw[c] = gm;
                float sg = 1.f;
#pragma unroll 4
                for (int i = W - 1; i >= 0; --i) {
                    Kt[i * KS + c] = Ap[i * KS + c] * sg;
                    sg *= Al[i * K + c];
                }
            }
        } else {
            // scalar decays: gamma_l = prod_{m<=l} alpha_m and sigma_l =
            // prod_{m>l} alpha_m for every slot at once (lane l of each DPP row
            // holds alpha_l: a prefix and a suffix product over the row); each
            // key chunk then takes its slot's pair from lane ki of its row
            float gam = as_l, sig = as_l;
            gam *= row_shr<1>(gam, 1.f);
            gam *= row_shr<2>(gam, 1.f);
            gam *= row_shr<4>(gam, 1.f);
            gam *= row_shr<8>(gam, 1.f);
            sig *= row_shl<1>(sig, 1.f);
            sig *= row_shl<2>(sig, 1.f);
            sig *= row_shl<4>(sig, 1.f);
            sig *= row_shl<8>(sig, 1.f);
            sig = row_shl<1>(sig, 1.f);
            gamW = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(gam), 0x150 + W - 1, 0xF, 0xF,
                                                              false));  // row_newbcast:15
            if (tid < KCH) {
                const float gi = __shfl(gam, ki, 16);
                const float si = __shfl(sig, ki, 16);
                float f[8], t[8];
                V8::unpack(kraw, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    f[e] = ki < n ? f[e] : 0.f;
                    t[e] = f[e] * si;
                }
                store8f(Kt + ki * KS + kc0, t);
                if (DELTA) {
                    store8f(Ap + ki * KS + kc0, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = f[e] * gi;
                    store8f(Kg + ki * KS + kc0, t);
                }
            }
        }
        __syncthreads();

        if (DELTA) {
            // 4a. L[i][l] = beta_i sum_c k_i[c] k_l[c] prod_{l<m<=i} alpha_m[c]
            // (l < i), row-major in Lr.  One DPP row of 16 lanes (channels
            // 8 l16 .. 8 l16 + 7 each) per entry.
            if (KDA) {
                // per-channel decays: row i walks l = i-1 .. 0, one more decay
                // per step (kd = k_i * prod_{l<m<=i} alpha_m).  With 32 DPP rows
                // or more the walk is split: row i takes l = i-1 .. i/2, row
                // W + i first applies the decays of slots i .. i/2 + 1 (cheap:
                // no sums) and then takes l = i/2 - 1 .. 0, so no row sums more
                // than eight entries; the products are formed in the same order.
                constexpr bool SPLIT = 4 * NW >= 2 * W;
                const int R = tid >> 4;
                const int l16 = tid & 15;
                const int i = SPLIT ? (R & (W - 1)) : R;
                const bool lower = SPLIT && R >= W;
                if (R < (SPLIT ? 2 * W : W) && i >= 1) {
                    const int h = SPLIT ? i / 2 : 0;
                    float kd[8];
                    load8f(Ap + i * KS + 8 * l16, kd);
                    const float bi = __shfl(bs_l, i, 16);
                    int jhi = i - 1, jlo = h;
                    if (lower) {
                        for (int m = i; m > h; --m) {
                            float am[8];
                            load8f(Al + m * K + 8 * l16, am);
#pragma unroll
                            for (int e = 0; e < 8; ++e) kd[e] *= am[e];
                        }
                        jhi = h - 1;
                        jlo = 0;
                    }
                    for (int j = jhi; j >= jlo; --j) {
                        float aj[8];
                        load8f(Al + (j + 1) * K + 8 * l16, aj);
#pragma unroll
                        for (int e = 0; e < 8; ++e) kd[e] *= aj[e];
                        float kj[8];
                        load8f(Ap + j * KS + 8 * l16, kj);
                        const float sum = row_sum16(dot8(kd, kj));
                        if (l16 == 0) Lr[i * 16 + j] = bi * sum;
                    }
                }
            } else {
                // scalar decays: L[i][l] = beta_i P[i][l] (k_i . k_l) with
                // P[i][l] = prod_{l<m<=i} alpha_m.  First every P[i][l] at
                // once, DPP row i lane l, as a suffix product over the lanes m > l
                // of the row (lanes above i contribute 1), with beta_i on the
                // diagonal; staged in the T area, whose solve comes later.
                float* Pm = Tm;
                if (tid < 16 * W) {
                    const int i = tid >> 4, l = tid & 15;  // lane l holds alpha_l, beta_l
                    float y = l <= i ? as_l : 1.f;
                    y *= row_shl<1>(y, 1.f);
                    y *= row_shl<2>(y, 1.f);
                    y *= row_shl<4>(y, 1.f);
                    y *= row_shl<8>(y, 1.f);  // prod_{m >= l, m <= i} alpha_m
                    const float pl = row_shl<1>(y, 1.f);
                    Pm[i * 16 + l] = l == i ? bs_l : pl;
                }
                __syncthreads();
                // then the W (W - 1) / 2 entries, spread over all 4 NW rows of
                // the block, a few per row
                const int row = tid >> 4;
                const int l16 = tid & 15;
                for (int p = row; p < W * (W - 1) / 2; p += 4 * NW) {
                    // p = i (i - 1) / 2 + j with 0 <= j < i
                    int i = int((1.f + __builtin_sqrtf(float(1 + 8 * p))) * 0.5f);
                    i = i * (i - 1) / 2 > p ? i - 1 : i;
                    i = (i + 1) * i / 2 <= p ? i + 1 : i;
                    const int j = p - i * (i - 1) / 2;
                    float ki[8], kj[8];
                    load8f(Ap + i * KS + 8 * l16, ki);
                    load8f(Ap + j * KS + 8 * l16, kj);
                    const float f = Pm[i * 16 + i] * Pm[i * 16 + j];
                    const float sum = row_sum16(dot8(ki, kj));
                    if (l16 == 0) Lr[i * 16 + j] = f * sum;
                }
            }
            __syncthreads();
            // 4b. T = (I + L)^{-1} diag(beta) by forward substitution, column c
            // by DPP row c: lane i holds T[i][c] and L's row i (zero above the
            // diagonal is never read); lane c starts from beta_c
            if (tid < 16 * W) {
                const int c = tid >> 4;
                const int l16 = tid & 15;
                float lrow[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v4 = *reinterpret_cast<const float4*>(Lr + l16 * 16 + 4 * q);
                    lrow[4 * q] = v4.x;
                    lrow[4 * q + 1] = v4.y;
                    lrow[4 * q + 2] = v4.z;
                    lrow[4 * q + 3] = v4.w;
                }
                float x = l16 == c ? bs_l : 0.f;
                TriSolveStep<0, W - 1>::run(x, lrow, l16);
                Tm[l16 * 16 + c] = x;
            }
            __syncthreads();
            // 4c. u = T V_w on this wave's columns, and -T (gamma K) over all keys
            float ta[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) ta[st] = Tm[lr * 16 + 4 * lq + st];
#pragma unroll
            for (int st = 0; st < 4; ++st) u = mfma_16x16x4(ta[st], Vw[(4 * lq + st) * VS + v0 + lr], u);
            for (int kt = w; kt < 8; kt += NW) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    d = mfma_16x16x4(ta[st], Kg[(4 * lq + st) * KS + 16 * kt + lr], d);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Ap[(4 * lq + rr) * KS + 16 * kt + lr] = -d[rr];
            }
            __syncthreads();
        }
        if (FUSED) {
            // With the state after the window S_n = P S_0 + X, P = M_W ... M_1 =
            // diag(gamma_W) - (sigma K)^T T (gamma K) and X = (sigma K)^T (T V_w)
            // (Mamba-2: P = gamma_W I, X = (sigma K)^T V_w), the last token's
            // buffered-token term is X^T q = (T V_w)^T w with w = (sigma K) q,
            // and its carried-back query is q~ = P^T q = gamma_W q - (gamma K)^T T^T w.
            {
                const int i = tid >> 4, l16 = tid & 15;
                if (i < W) {
                    float k8[8], q8[8];
                    load8f(Kt + i * KS + 8 * l16, k8);
                    load8f(Qs + 8 * l16, q8);
                    const float wi = row_sum16(dot8(k8, q8));
                    if (l16 == 0) Ws[i] = wi;
                }
            }
            __syncthreads();
            // this lane's column of X^T q: its four token rows 4 lq + rr
            {
                float ip = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    ip = fmaf(Ws[4 * lq + rr], DELTA ? u[rr] : Vw[(4 * lq + rr) * VS + v0 + lr], ip);
                intra = quarter_sum4(ip);
            }
            if (DELTA && sketch) {
                if (tid < W) {
                    float t = 0.f;
#pragma unroll
                    for (int i = 0; i < W; ++i) t = fmaf(Tm[i * 16 + tid], Ws[i], t);
                    Ts[tid] = t;
                }
                __syncthreads();
                if (tid < K) {
                    float x = (KDA ? Gw[tid] : gamW) * Qs[tid];
#pragma unroll
                    for (int i = 0; i < W; ++i) x = fmaf(-Ts[i], Kg[i * KS + tid], x);
                    Qt[tid] = x;
                }
                __syncthreads();
            }
            if (sketch) {
                // c = F q~ for map rows 0 .. 15 (the tile landed with the window
                // and the window barriers made it visible), then this lane's
                // part of sum_m c_m Z_old[m][column]
                {
                    const int m = tid >> 4, l16 = tid & 15;
                    if (m < 16) {
                        float f8[8], q8[8];
                        load8f(Fm + m * K + 8 * l16, f8);
                        load8f((DELTA ? Qt : Qs) + 8 * l16, q8);
                        float cm = row_sum16(dot8(f8, q8));
                        if (!DELTA) cm *= gamW;
                        if (l16 == 0) Cs[m] = cm;
                    }
                }
                __syncthreads();
                float zp = 0.f;
#pragma unroll
                for (int jz = 0; jz < 4; ++jz)
                    if (lq + 4 * jz < r) zp = fmaf(Cs[lq + 4 * jz], zo[jz], zp);
                zc = quarter_sum4(zp);
            }
        }
    }
    // nothing that reads the state may be scheduled above this point
    __builtin_amdgcn_sched_barrier(0);

    // ---- 5. with the state: U and the update ----
    if (n > 0) {
        if (DELTA) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(Ap + lr * KS + 16 * kt + 4 * lq);
#pragma unroll
                for (int ss = 0; ss < 4; ++ss) u = mfma_16x16x4(a4[ss], s[kt][ss], u);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            f32x4 acc;
            if (KDA) {
                const f32x4 g4 = *reinterpret_cast<const f32x4*>(Gw + 16 * kt + 4 * lq);
                acc = g4 * s[kt];
            } else {
                acc = gamW * s[kt];
            }
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) {
                const float bop = DELTA ? u[ss] : Vw[(4 * lq + ss) * VS + v0 + lr];
                acc = mfma_16x16x4(Kt[(4 * lq + ss) * KS + 16 * kt + lr], bop, acc);
            }
            s[kt] = acc;
        }
    }
    // fused: the last token's output.  A dense head reads S_n^T q exactly; a
    // sketch head outputs Z_old^T (F q~) + X^T q (both formed above while the
    // state was in flight, plus the map tiles beyond the first).
    if (FUSED) {
        float yv;
        if (sketch) {
            for (int mt = 1; 16 * mt < r; ++mt) {  // ranks above 16
                __syncthreads();  // every row is done with the previous tile
                stage_fmap(mt);
                float zm[4];
#pragma unroll
                for (int jz = 0; jz < 4; ++jz)
                    zm[jz] = Zold[size_t(min(16 * mt + lq + 4 * jz, r - 1)) * V + v0 + lr];
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile and the rows
                __syncthreads();
                {
                    const int m = tid >> 4, l16 = tid & 15;
                    if (m < 16) {
                        float f8[8], q8[8];
                        load8f(Fm + m * K + 8 * l16, f8);
                        load8f((DELTA ? Qt : Qs) + 8 * l16, q8);
                        float cm = row_sum16(dot8(f8, q8));
                        if (!DELTA) cm *= gamW;
                        if (l16 == 0) Cs[m] = cm;
                    }
                }
                __syncthreads();
                float zp = 0.f;
#pragma unroll
                for (int jz = 0; jz < 4; ++jz)
                    if (16 * mt + lq + 4 * jz < r) zp = fmaf(Cs[lq + 4 * jz], zm[jz], zp);
                zc += quarter_sum4(zp);
            }
            yv = zc + intra;
        } else {
            float yp = 0.f;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                const f32x4 q4 = *reinterpret_cast<const f32x4*>(Qs + 16 * kt + 4 * lq);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) yp = fmaf(s[kt][rr], q4[rr], yp);
            }
            yv = quarter_sum4(yp);
        }
        if (lq == 0) A.y[item * V + v0 + lr] = yv;
    }
    // ---- 6. Z = Omega_r S for a sketch head, then the state store ----
    // Z goes first: storing the state first needs no extra wait either, but
    // measured slower (the block's stores then trail its Z work).  Every wave
    // waited for its own first-tile basis granules before its state load; the
    // first window barrier (or the one below when there is no window) makes
    // all of them visible.  The two cases keep separate tails so that no path
    // reaches the stores with a state load the compiler still counts as
    // outstanding.
    auto sketch_rows = [&]() {
        float* Zi = A.Z + (size_t(T.zrow[p]) * A.B + size_t(b) * r) * V;
        const int mts = (r + 15) >> 4;
        for (int mt = 0; mt < mts; ++mt) {
            if (mt > 0) {
                // ranks above 16: the next tile replaces the last one (a cache
                // hit: the head's blocks run back to back)
                __syncthreads();
                stage_basis(mt);
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's granules
                __syncthreads();
            }
            const float* orow = Om + lr * K;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                const f32x4 o = *reinterpret_cast<const f32x4*>(orow + 4 * ((4 * kt + lq) ^ lr));
#pragma unroll
                for (int ss = 0; ss < 4; ++ss) z = mfma_16x16x4(o[ss], s[kt][ss], z);
            }
            if (DELTA) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int m = 16 * mt + 4 * lq + rr;
                    if (m < r) Zi[size_t(m) * V + v0 + lr] = z[rr];
                }
            } else {
                // whole sketch rows through the dead window-phase LDS, as the state
                static_assert(16 * VS <= L::om, "sketch tile overlaps the basis tile");
                __syncthreads();  // every wave is past the update and the last tile's reads
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sm[(4 * lq + rr) * VS + v0 + lr] = z[rr];
                __syncthreads();
                const int rows = min(16, r - 16 * mt);
                const int row = tid / (V / 4), c4 = tid - row * (V / 4);  // 4 V threads: one piece each
                if (row < rows)
                    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sm + row * VS + 4 * c4),
                                                reinterpret_cast<f32x4*>(Zi + size_t(16 * mt + row) * V + 4 * c4));
            }
        }
    };
    if (n > 0) {
        if (sketch) sketch_rows();
        if (DELTA) {
            // staging the state through LDS measured no faster for the
            // delta-rule kernels (eight waves, three blocks per CU)
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) buffer_store_f32(s[kt][rr], srs, svo, (16 * kt + rr) * V * 4);
        } else {
            // whole rows through the window-phase LDS (keys and values), dead
            // once every wave has applied the update; streaming stores, as for
            // the sketch rows (a little faster: neither is read again before
            // the next flush)
            static_assert(2 * 16 * VS <= L::om, "state tiles overlap the basis tile");
            store_state_tiles<V, 16, 2, true>(s, sm, srs, tid);
        }
    } else if (sketch) {
        __syncthreads();
        sketch_rows();
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int KIND, int V, typename QT, bool FUSED>
static hipError_t launch_flush_f(const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    const size_t lds = FlushLds<KIND, V, FUSED>::bytes(a.omt);
    auto fn = flush_kernel<KIND, V, QT, FUSED>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(V / 16 * 64), lds, s, a, t);
    return hipGetLastError();
}

template <int KIND, int V, typename QT>
static hipError_t launch_flush_t(const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    if (!a.y) return launch_flush_f<KIND, V, QT, false>(a, t, grid, s);
    return launch_flush_f<KIND, V, QT, true>(a, t, grid, s);
}

template <int KIND, typename QT>
static hipError_t launch_flush_v(int V, const FlushArgs& a, const HeadTable& t, int grid,
                                 hipStream_t s) {
    switch (V) {
        case 64: return launch_flush_t<KIND, 64, QT>(a, t, grid, s);
        case 80: return launch_flush_t<KIND, 80, QT>(a, t, grid, s);
        case 96: return launch_flush_t<KIND, 96, QT>(a, t, grid, s);
        case 112: return launch_flush_t<KIND, 112, QT>(a, t, grid, s);
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

// The fused last read's extra arguments (null for a plain flush).
struct FusedRead {
    const float* frames;
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* beta;
    float* y;
};

static sketchssm_status run_flush(const sketchssm_plan* plan, float* S, float* Z,
                                  const float* basis, const void* kbuf, const void* vbuf,
                                  const float* abuf, const float* bbuf, int32_t n_tokens,
                                  const int32_t* seqs, const int32_t* ntok, int32_t n_seqs,
                                  void* stream, const FusedRead* fr = nullptr) {
    if (!plan) return SKSSM_EINVAL;
    const sketchssm_shape& sh = plan->shape;
    const bool delta = sh.kind != SKSSM_MAMBA2;
    const int n_sketch = sh.H - plan->n_dense;
    const bool listed = seqs != nullptr;
    // with a list every count is on the device: the window must be there
    const bool window = listed ? n_seqs > 0 : n_tokens > 0;
    if (!S) return SKSSM_EINVAL;
    if (!listed && (n_tokens < 0 || n_tokens > sh.W)) return SKSSM_EINVAL;
    if (listed && (!ntok || n_seqs < 0)) return SKSSM_EINVAL;
    if (n_sketch > 0 && (!Z || !basis)) return SKSSM_EINVAL;
    if (window && (!kbuf || !vbuf || !abuf)) return SKSSM_EINVAL;
    if (window && delta && !bbuf) return SKSSM_EINVAL;
    if (!delta && bbuf) return SKSSM_EINVAL;
    const void* ptrs[] = {S, Z, basis, kbuf, vbuf, abuf, bbuf};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return SKSSM_EALIGN;
    if (listed && ((reinterpret_cast<uintptr_t>(seqs) | reinterpret_cast<uintptr_t>(ntok)) & 3u))
        return SKSSM_EALIGN;
    if (fr) {
        if (!fr->q || !fr->k || !fr->v || !fr->a || !fr->y) return SKSSM_EINVAL;
        if (delta != (fr->beta != nullptr)) return SKSSM_EINVAL;
        if (n_sketch > 0 && !fr->frames) return SKSSM_EINVAL;
        const void* fptrs[] = {fr->frames, fr->q, fr->k, fr->v, fr->a, fr->beta, fr->y};
        for (const void* ptr : fptrs)
            if (ptr && !aligned16(ptr)) return SKSSM_EALIGN;
    }
    if (listed && n_seqs == 0) return SKSSM_OK;
    if (!listed && n_sketch == 0 && n_tokens == 0) return SKSSM_OK;  // nothing to write

    FlushArgs A;
    A.S = S;
    A.Z = n_sketch > 0 ? Z : nullptr;
    A.basis = basis;
    A.kbuf = kbuf;
    A.vbuf = vbuf;
    A.abuf = abuf;
    A.bbuf = bbuf;
    A.seqs = seqs;
    A.ntok = ntok;
    A.B = sh.B;
    A.H = sh.H;
    A.n_tokens = listed ? 0 : n_tokens;
    A.basis_rows = sh.basis_rows;
    A.nb = listed ? n_seqs : sh.B;
    A.Hk = kq_heads_of(sh);
    A.share = sh.H / A.Hk;
    A.omt = n_sketch > 0 ? 1 : 0;
    A.tq = fr ? fr->q : nullptr;
    A.tk = fr ? fr->k : nullptr;
    A.tv = fr ? fr->v : nullptr;
    A.ta = fr ? fr->a : nullptr;
    A.tb = fr ? fr->beta : nullptr;
    A.frames = fr ? fr->frames : nullptr;
    A.y = fr ? fr->y : nullptr;
    const long grid = long(A.nb) * sh.H;
    if (grid > 0x7fffffffL) return SKSSM_ESHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = sh.qkv == SKSSM_BF16
                             ? launch_flush_k<Bf16Tag>(sh.kind, sh.V, A, plan->table, int(grid), s)
                             : launch_flush_k<F32Tag>(sh.kind, sh.V, A, plan->table, int(grid), s);
    return e == hipSuccess ? SKSSM_OK : SKSSM_ELAUNCH;
}

extern "C" sketchssm_status sketchssm_flush(const sketchssm_plan* plan, float* S, float* Z,
                                            const float* basis, const void* kbuf,
                                            const void* vbuf, const float* abuf,
                                            const float* bbuf, int32_t n_tokens, void* stream) {
    return run_flush(plan, S, Z, basis, kbuf, vbuf, abuf, bbuf, n_tokens, nullptr, nullptr, 0,
                     stream);
}

extern "C" sketchssm_status sketchssm_flush_seq(const sketchssm_plan* plan, float* S, float* Z,
                                                const float* basis, const void* kbuf,
                                                const void* vbuf, const float* abuf,
                                                const float* bbuf, const int32_t* seqs,
                                                const int32_t* n_tokens, int32_t n_seqs,
                                                void* stream) {
    if (!seqs) return SKSSM_EINVAL;
    return run_flush(plan, S, Z, basis, kbuf, vbuf, abuf, bbuf, 0, seqs, n_tokens, n_seqs, stream);
}

extern "C" sketchssm_status sketchssm_decode_read_flush(const sketchssm_plan* plan, float* S, float* Z,
                                                       const float* frames, const float* basis,
                                                       const void* q, const void* k, const void* v,
                                                       const float* a, const float* beta, void* kbuf,
                                                       void* vbuf, float* abuf, float* bbuf, float* y,
                                                       void* stream) {
    if (!plan) return SKSSM_EINVAL;
    const FusedRead fr{frames, q, k, v, a, beta, y};
    return run_flush(plan, S, Z, basis, kbuf, vbuf, abuf, bbuf, plan->shape.W, nullptr, nullptr, 0,
                     stream, &fr);
}
