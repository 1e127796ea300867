/*
 * sketchssm.h -- C ABI of the SketchSSM decode hot path for MI355X (gfx950).
 *
 * SketchSSM writes every update of a linear-attention / SSM head's recurrent
 * state in full, and in the stretch between two exact flushes it serves decode
 * queries from a small low-rank summary of the state rather than the state
 * (page "SketchSSM" (PyPI, sketchssm 0.1.0), opening paragraph; page
 * "SketchSSM: Write to the Full State, Read from a Compact Sketch", Abstract).
 *
 * Per (batch b, head h) "item" with key dim K and value dim V:
 *   state     S in R^{K x V}, fp32 (the PyPI page's serving command keeps the
 *             recurrent state cache in float32, "Quick start: serve with vLLM");
 *   basis     Omega_g in R^{basis_rows x K}, one per head group; a head of rank
 *             r uses its first r rows (calibration card "SketchSSM calibration:
 *             Nemotron Nano 9B v2", "Contents": basis (27, 8, 79, 128));
 *   frame     the coefficient map F in R^{r x K} of one (group, rank) pair;
 *   sketch    Z = Omega_r S in R^{r x V}, formed at a flush, the one point where
 *             the full state is read (Abstract: the basis directions' outputs are
 *             kept from each state update);
 *   window    the W tokens (k, v, decay, beta) held back since the last flush
 *             (Abstract: updates are amortised by holding keys and values back;
 *             W = 16 on the card).
 * Transitions: Mamba-2  M = a I;  Gated DeltaNet  M = alpha (I - beta k k^T);
 * KDA  M = (I - beta k k^T) diag(alpha).  Update S_t = M_t S_{t-1} + beta k v^T
 * (beta = 1 for Mamba-2).  At window position j the output is
 *   sketch head:  y = Z^T (F q~) + intra,   dense head:  y = S_0^T q~ + intra,
 * with q~ = M_1^T ... M_j^T q (the query carried back through the window) and
 * intra the exact contribution of the buffered tokens; S_0 is the state at the
 * last flush.
 *
 * Conventions for every call below:
 *   - "device" pointers are HIP device allocations owned by the caller; the
 *     library never allocates, frees or synchronises on the launch path;
 *   - every device pointer must be 16-byte aligned (SKSSM_EALIGN otherwise);
 *   - calls are asynchronous on `stream` (a hipStream_t; NULL = null stream);
 *   - arguments are checked on the host before anything is launched and a
 *     status is returned; nothing throws across this boundary;
 *   - all arrays are dense row-major with the layouts written beside them.
 * Supported shapes: K = 128, W = 16, V a multiple of 16 from 64 to 128 (the
 * Nano layer's 80, GDN/KDA's 128), 1 <= H <= 256,
 * rank_cap <= 64.  Below, Hk = kq_heads (or H when 0) and head h uses key/query
 * head h / (H / Hk).
 */
#ifndef SKETCHSSM_H
#define SKETCHSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKSSM_OK = 0,
    SKSSM_EINVAL = 1,   /* null pointer, bad enum, pos / n_tokens out of range */
    SKSSM_ESHAPE = 2,   /* unsupported or inconsistent shape, rank out of range */
    SKSSM_EALIGN = 3,   /* a device pointer is not 16-byte aligned */
    SKSSM_ENOMEM = 4,   /* host allocation of a plan failed */
    SKSSM_EDEVICE = 5,  /* HIP runtime error before launch */
    SKSSM_ELAUNCH = 6   /* hipGetLastError reported a launch failure */
} sketchssm_status;

typedef enum {
    SKSSM_MAMBA2 = 0,   /* scalar decay a, no erase (card "Contents": erase factor no) */
    SKSSM_GDN = 1,      /* scalar decay alpha, delta-rule erase with beta */
    SKSSM_KDA = 2       /* per-channel decay alpha in R^K, delta-rule erase */
} sketchssm_kind;

typedef enum {
    SKSSM_BF16 = 0,     /* q, k, v and the window's k, v in bfloat16 */
    SKSSM_F32 = 1       /* q, k, v and the window's k, v in float32 */
} sketchssm_dtype;

/* One layer's state, B * H * K * V fp32 elements, must stay below 2^31 (8 GiB):
 * up to 1638 sequences at 128 heads of 128 x 80.  Larger shapes give SKSSM_ESHAPE. */
typedef struct {
    int32_t B;          /* batch (sequences) */
    int32_t H;          /* state heads of the layer */
    int32_t K;          /* key dim (128) */
    int32_t V;          /* value dim: 64, 80, 96, 112 or 128 */
    int32_t W;          /* window length between flushes (16) */
    int32_t G;          /* basis groups */
    int32_t basis_rows; /* rows per group basis (79 on the Nano card) */
    int32_t rank_cap;   /* largest allowed rank (49 on the Nano card; <= 64) */
    int32_t kind;       /* sketchssm_kind */
    int32_t qkv;        /* sketchssm_dtype */
    int32_t kq_heads;   /* heads of q and k: each is shared by H / kq_heads consecutive
                           state heads (grouped keys and queries, as a Mamba-2 layer's
                           B and C are per group); 0 or H = one per head.  Must divide H. */
} sketchssm_shape;

typedef struct sketchssm_plan sketchssm_plan;   /* opaque, immutable once made */

/*
 * Host only (no HIP call).  Checks the shape and the rank table and derives the
 * frames and the launch order (the calibration card obtains each head's rank
 * and the frame order from its allocation scores for whatever mean rank is
 * asked for; card "SketchSSM calibration: Nemotron Nano 9B v2", opening
 * paragraph).
 *   rank[H]  : 0 = dense fallback, else 1 <= rank <= min(rank_cap, basis_rows, K)
 *   group[H] : basis group of each head, 0 <= group < G
 * Frames are the distinct (group, rank) pairs of the sketch heads sorted by
 * group then rank; bucket[h] = 0 (dense) or 1 + (rank-1)/8; the order lists
 * dense heads first, then buckets from high to low, heads ascending within a
 * bucket.  The decode read launches the sketch heads' tiles in that order and
 * the dense heads' items after them (a dense item's block moves fewer bytes
 * than a 16-row sketch tile's).  Both arrays are copied; *out receives a plan
 * to free with sketchssm_plan_destroy.  A plan may be shared by threads and
 * streams.
 */
sketchssm_status sketchssm_plan_create(const sketchssm_shape* shape, const int32_t* rank,
                                       const int32_t* group, sketchssm_plan** out);

/*
 * Host only.  As sketchssm_plan_create, with the launch order given instead of
 * derived (the pages fix no order; this serves to compare orders, e.g. head
 * order against the rank buckets):
 *   order[H] : a permutation of 0..H-1 listing every dense head (rank 0) before
 *              any sketch head; copied.
 * Frames, offsets and buckets are those of sketchssm_plan_create; only the
 * launch order differs, and no result depends on it (every item is computed
 * the same way in any order).  SKSSM_ESHAPE if order is not such a permutation.
 */
sketchssm_status sketchssm_plan_create_ordered(const sketchssm_shape* shape, const int32_t* rank,
                                               const int32_t* group, const int32_t* order,
                                               sketchssm_plan** out);

/*
 * Host only.  Copies the derived tables into caller arrays (any may be NULL):
 *   frame_index[H]    frame of each head, -1 for a dense head
 *   frame_row_off[F+1] first row of each frame in the frames array
 *   z_row_off[H+1]    running sum of the heads' ranks
 *   bucket[H], order[H]
 *   frame_group[F], frame_rank[F]  the (group, rank) of each frame
 *   n_frames          F
 */
sketchssm_status sketchssm_plan_export(const sketchssm_plan* plan, int32_t* frame_index,
                                       int32_t* frame_row_off, int32_t* z_row_off,
                                       int32_t* bucket, int32_t* order, int32_t* frame_group,
                                       int32_t* frame_rank, int32_t* n_frames);

void sketchssm_plan_destroy(sketchssm_plan* plan);

/* fp32 elements of the sketch array: B * V * sum_h rank[h].
 * Layout: Z[((z_row_off[h] * B) + b * rank[h] + i) * V + v], i < rank[h]. */
size_t sketchssm_z_elems(const sketchssm_plan* plan);

/* fp32 elements of the frames array: K * sum_f rank_f.
 * Layout: frames[(frame_row_off[f] + i) * K + k], i < rank_f (the map F of frame f). */
size_t sketchssm_frame_elems(const sketchssm_plan* plan);

/*
 * Flush: apply window slots 0 .. n_tokens-1 to the state and, in the same pass
 * over S, write the sketch Z = Omega_r S of every sketch head (Abstract: S is
 * read a single time per update and its products with the basis are stored).
 *   S      device [B,H,K,V] fp32, in/out.  n_tokens = 0 leaves S bitwise
 *          unchanged and only writes Z (the initial sketch after prefill);
 *          dense heads' states are then not even read.
 *   Z      device [sketchssm_z_elems] fp32, out; may be NULL when no head has a rank
 *   basis  device [G, basis_rows, K] fp32
 *   kbuf   device [W,Hk,B,K] of the qkv dtype     (window keys)
 *   vbuf   device [W,H,B,V] of the qkv dtype      (window values)
 *   abuf   device [W,H,B] fp32 (Mamba-2, GDN) or [W,H,B,K] fp32 (KDA) (decays)
 *   bbuf   device [W,H,B] fp32 (GDN, KDA); must be NULL for Mamba-2
 *          The window is slot-major: slot i of item (b, h) is element
 *          (i*H + h)*B + b of vbuf, abuf, bbuf and (i*Hk + h/(H/Hk))*B + b of
 *          kbuf; a shared key slot is written once, by the first of its heads.
 *          A decode step then appends one contiguous slab and reads older
 *          slots as contiguous runs of batch rows.
 *   n_tokens 0 .. W
 * The window is not modified; the next window simply starts again at slot 0.
 */
sketchssm_status sketchssm_flush(const sketchssm_plan* plan, float* S, float* Z,
                                 const float* basis, const void* kbuf, const void* vbuf,
                                 const float* abuf, const float* bbuf, int32_t n_tokens,
                                 void* stream);

/*
 * Decode read of one token at window position pos (0-based; the token is the
 * (pos+1)-th since the last flush).  Appends the token to window slot pos, sweeps
 * the window back to the flush to form q~ and the buffered tokens' exact term,
 * then outputs y = Z^T (F q~) + intra for sketch heads and y = S_0^T q~ + intra
 * for dense heads (Abstract: a decode step mixes the stored sketch rows with
 * weights computed from the query and leaves S untouched; PyPI page, "Make a
 * calibration for your model": a head gets a rank or a dense fallback).  Sketch
 * heads never read S.
 *   S       device [B,H,K,V] fp32 state at the last flush (read by dense heads only)
 *   Z       device sketch (see sketchssm_z_elems); may be NULL without sketch heads
 *   frames  device [sketchssm_frame_elems] fp32; may be NULL without sketch heads
 *   q, k    device [B,Hk,K] qkv dtype
 *   v       device [B,H,V] qkv dtype
 *   a       device [B,H] fp32 (Mamba-2, GDN) or [B,H,K] fp32 (KDA)
 *   beta    device [B,H] fp32 (GDN, KDA); NULL for Mamba-2
 *   kbuf, vbuf, abuf, bbuf   the window (layouts as in sketchssm_flush); slot pos
 *           is written, slots < pos are read
 *   pos     0 .. W-1
 *   y       device [B,H,V] fp32, out
 * After the read at pos = W-1 the caller runs sketchssm_flush(n_tokens = W) on the
 * same stream.
 */
sketchssm_status sketchssm_decode_read(const sketchssm_plan* plan, const float* S,
                                       const float* Z, const float* frames, const void* q,
                                       const void* k, const void* v, const float* a,
                                       const float* beta, void* kbuf, void* vbuf, float* abuf,
                                       float* bbuf, int32_t pos, float* y, void* stream);

/*
 * Continuous batching: sketchssm_decode_read where every sequence has its own
 * window position (sequences join, flush and leave at different steps).
 *   pos     device [B] int32: row b reads and appends at window slot pos[b]
 *           (0 .. W-1); any other value (e.g. -1) leaves the row idle -- nothing
 *           of it is read or written and y keeps its previous contents.  The
 *           array is read on the device, so bad values are not reported; they
 *           only idle the row.
 * Other arguments as in sketchssm_decode_read.  The caller flushes a row with
 * sketchssm_flush_seq after its read at pos[b] = W-1 and restarts it at 0.
 */
sketchssm_status sketchssm_decode_read_seq(const sketchssm_plan* plan, const float* S,
                                           const float* Z, const float* frames, const void* q,
                                           const void* k, const void* v, const float* a,
                                           const float* beta, void* kbuf, void* vbuf,
                                           float* abuf, float* bbuf, const int32_t* pos, float* y,
                                           void* stream);

/*
 * Per-sequence flush: sketchssm_flush for the listed batch rows only.
 *   seqs      device [n_seqs] int32: batch rows, each at most once per call
 *             (two blocks updating one row's state would race)
 *   n_tokens  device [n_seqs] int32: held-back tokens of that row's window,
 *             0 .. W (W after a full window; fewer to close a window early;
 *             0 after a prefill, forming the row's first sketch with S untouched)
 *   n_seqs    >= 0; 0 does nothing
 * kbuf, vbuf, abuf (and bbuf for the delta rule) are required even if every
 * count is 0, since the counts live on the device.  A listed row outside
 * 0 .. B-1 or a count outside 0 .. W idles that row's blocks.
 */
sketchssm_status sketchssm_flush_seq(const sketchssm_plan* plan, float* S, float* Z,
                                     const float* basis, const void* kbuf, const void* vbuf,
                                     const float* abuf, const float* bbuf, const int32_t* seqs,
                                     const int32_t* n_tokens, int32_t n_seqs, void* stream);

/*
 * The window's last read and its flush in one pass: equivalent to
 * sketchssm_decode_read at pos = W-1 followed by sketchssm_flush(n_tokens = W)
 * on the same stream, with the same outputs.  The flush already holds the
 * state at the last flush, the updated state and the window, so the token's
 * carried-back query q~ = (M_W ... M_1)^T q comes from the chunked form of the
 * update, and the sketch read is Z_old^T (F q~) + (S_n^T q - S_0^T q~), the
 * bracket being the buffered tokens' exact term (Abstract of "SketchSSM: Write
 * to the Full State, Read from a Compact Sketch": buffered keys and values,
 * reads from the stored sketch; dense heads output S_n^T q).  The window's
 * slots 0 .. W-2 are read; the current token is taken from q, k, v, a, beta
 * (the window restarts at slot 0 afterwards).  One pass for every layer kind.
 *   S, Z          as in sketchssm_flush (Z is read as the old sketch, then
 *                 overwritten with the new one)
 *   frames        as in sketchssm_decode_read; basis as in sketchssm_flush
 *   q, k, v, a, beta, y   as in sketchssm_decode_read
 *   kbuf .. bbuf  the window: slots 0 .. W-2 are read; slot W-1 may be written
 */
sketchssm_status sketchssm_decode_read_flush(const sketchssm_plan* plan, float* S, float* Z,
                                             const float* frames, const float* basis,
                                             const void* q, const void* k, const void* v,
                                             const float* a, const float* beta, void* kbuf,
                                             void* vbuf, float* abuf, float* bbuf, float* y,
                                             void* stream);

/*
 * Full-state-read baseline: sketchssm_decode_read with every head dense (each
 * query reads S_0; the ReplaySSM-style read that the Abstract contrasts with).
 * Arguments as in sketchssm_decode_read; the shape replaces the plan.
 */
sketchssm_status sketchssm_dense_read(const sketchssm_shape* shape, const float* S,
                                      const void* q, const void* k, const void* v,
                                      const float* a, const float* beta, void* kbuf,
                                      void* vbuf, float* abuf, float* bbuf, int32_t pos,
                                      float* y, void* stream);

/*
 * Standard per-token decode, the baseline that the pages quote their kernel
 * speedups against ("SketchSSM: Write to the Full State, Read from a Compact
 * Sketch", Abstract: the standard vLLM decode; read here as the plain
 * recurrence, which reads and writes the whole state for every token).  For
 * every (b, h): S <- M S + beta k v^T, then y = S^T q (the updated state).
 * No window, plan, sketch or basis is involved.
 *   S       device [B,H,K,V] fp32, in/out
 *   q, k    device [B,Hk,K] qkv dtype;  v device [B,H,V] qkv dtype
 *   a       device [B,H] fp32 (Mamba-2, GDN) or [B,H,K] fp32 (KDA)
 *   beta    device [B,H] fp32 (GDN, KDA); NULL for Mamba-2
 *   y       device [B,H,V] fp32, out
 */
sketchssm_status sketchssm_rmw_step(const sketchssm_shape* shape, float* S, const void* q,
                                    const void* k, const void* v, const float* a,
                                    const float* beta, float* y, void* stream);

/* Static English text for a status code. */
const char* sketchssm_status_string(sketchssm_status status);

#ifdef __cplusplus
}
#endif

#endif /* SKETCHSSM_H */
