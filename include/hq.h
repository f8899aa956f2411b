/*
 * hq.h -- C ABI of the HyQuant hybrid-precision attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes (pages about "HyQuant: Hybrid-Precision
 * Quantization for LLM Attention", cited by page and section):
 *   [AFS] "HyQuant ... Explained for Beginners" (aifromscratch.in),
 *         "How It Works: The Hybrid-Precision Strategy" and
 *         "The Technical Mechanics: Two Operational Modes".
 *   [WPN] "Hybrid-precision attention reduces compute cost with minimal
 *         accuracy loss" (wpnews.pro), body paragraph 4.
 *   [KQ]  kipquest.com paper page 2608.27875, "The abstract".
 *   [HP]  hotpaper.ai paper page 2608.27875, technical-approach list.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless a comment says "host".
 *  - The caller allocates and frees every buffer, workspaces included; the
 *    library never allocates device memory and keeps no pointer after a call
 *    returns.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *    work; buffers must stay alive until the stream has reached it.
 *  - Every host-checkable precondition is validated before anything is
 *    enqueued. On failure the call returns a non-zero hq_status, enqueues
 *    nothing, and hq_last_error() gives a message (thread local). A failed
 *    launch returns HQ_ERR_HIP. No C++ exception crosses this boundary.
 *  - Device-side preconditions that are NOT checked: inputs are finite and
 *    the fp16 scale/zero of every group is finite (|x| <= 65504); index lists
 *    are strictly ascending where stated.
 *  - Results are deterministic: same inputs, same sizes, same device =>
 *    bitwise identical outputs (no floating-point atomics, fixed merge order).
 *
 * INT4 storage (the pages say only "4-bit keys and values" [AFS, How It
 * Works, item 3]; the format is this library's reading): per token and per
 * group of `group` = 32 consecutive channels, codes c in 0..15 with
 * x_hat = c * s + z, s = fp16((max - min) / 15), z = fp16(min), c =
 * clamp(rint_even((x - z) / s), 0, 15) in fp32, s = 0 and c = 0 for a
 * constant group. Two planes per head:
 *  - codes, HQ_LAYOUT_ROWS: [rows][D/2] bytes, byte j of a row holds channel
 *    2j in its low nibble and channel 2j+1 in its high nibble (used for K).
 *  - codes, HQ_LAYOUT_TILE16: rows grouped in tiles of 16; tile u is a
 *    [D/2][16] byte block: byte (j, 4a + b) holds channels 2j (low nibble)
 *    and 2j+1 (high nibble) of row 16u + 4a + (0, 2, 1, 3)[b] (used for V:
 *    one 16-byte load gives one channel pair of 16 consecutive tokens, and
 *    each 32-bit word holds rows (t, t+1) in its even bytes and (t+2, t+3) in
 *    its odd bytes). The row capacity of a TILE16 plane is a multiple of 16.
 *  - scale/zero: [rows][D/group][2] fp16 bit patterns {scale, zero}.
 */
#ifndef HQ_H_
#define HQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_ABI_VERSION 3

/* Each enum below carries two range markers (never returned or accepted) so
 * that every int is a representable value of the type: a caller passing an
 * unknown value gets HQ_ERR_INVALID_ARG (or "unknown status") instead of
 * undefined behaviour in the library. */
typedef enum {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARG = 1,   /* a null pointer, a size or range out of bounds */
  HQ_ERR_UNSUPPORTED = 2,   /* a valid but unimplemented shape or dtype */
  HQ_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  HQ_ERR_HIP = 4,           /* the HIP runtime reported an error */
  HQ_STATUS_RANGE_LO_ = -2147483647 - 1,
  HQ_STATUS_RANGE_HI_ = 2147483647
} hq_status;

typedef enum {
  HQ_F32 = 0, HQ_BF16 = 1, HQ_F16 = 2,
  HQ_DTYPE_RANGE_LO_ = -2147483647 - 1, HQ_DTYPE_RANGE_HI_ = 2147483647
} hq_dtype;

typedef enum {
  HQ_LAYOUT_ROWS = 0, HQ_LAYOUT_TILE16 = 1,
  HQ_LAYOUT_RANGE_LO_ = -2147483647 - 1, HQ_LAYOUT_RANGE_HI_ = 2147483647
} hq_code_layout;

/* Detector forms: the pages' matrix multiplication (MFMA) followed by
 * column sums, or the same scores through the sum of the query rows followed
 * by one matrix-vector product (equal by linearity). */
typedef enum {
  HQ_DETECT_MATMUL = 0, HQ_DETECT_QSUM = 1,
  HQ_DETECT_RANGE_LO_ = -2147483647 - 1, HQ_DETECT_RANGE_HI_ = 2147483647
} hq_detect_method;

/*
 * One layer's hybrid KV cache for a decode step [AFS, How It Works: the
 * three token sets; Technical Mechanics, Decode Stage]. Caller owned.
 * Positions [0, T) split into:
 *   Win = [T - W, T)   local window (current token included), 16-bit rows;
 *   VL  = a set of k positions inside [0, T - W), 16-bit rows;
 *   the rest of [0, T - W), INT4 rows from the planes.
 * The VL set is given twice, in the two forms the kernel reads: the compact
 * rows vl_k / vl_v (row i = the i-th VL position in ascending order, built by
 * hq_gather_rows) and the membership bitmap vl_bits (built by hq_vl_bitmap
 * from the same index list). The INT4 planes cover at least [0, T - W); rows
 * at VL positions may hold anything: they never reach the result.
 */
typedef struct {
  int B, Hkv, D, group;       /* D in {64, 128}; group = 32 */
  int64_t T;                  /* context length including the current token */
  int W;                      /* window length, 0 <= W <= T */
  int k;                      /* VL rows per (b, h), 0 <= k <= T - W */
  int64_t t_cap;              /* row capacity of the INT4 planes: >= T - W and
                                 a multiple of 32 */
  const uint8_t *k_codes;     /* HQ_LAYOUT_ROWS   [B][Hkv][t_cap][D/2] */
  const uint8_t *v_codes;     /* HQ_LAYOUT_TILE16 [B][Hkv][t_cap/16][D/2][16] */
  const uint16_t *k_sz;       /* [B][Hkv][t_cap][D/group][2] fp16 {s, z} */
  const uint16_t *v_sz;       /* [B][Hkv][t_cap][D/group][2] fp16 {s, z} */
  const uint32_t *vl_bits;    /* [B][Hkv][t_cap/32]: bit t%32 of word t/32 set
                                 iff position t is a VL position */
  const void *vl_k, *vl_v;    /* [B][Hkv][k][D] hp_dtype, the VL rows (ascending
                                 position order as gathered from a detector's list,
                                 any order after hq_vl_update: the attention reads
                                 them as a set) */
  const void *win_k, *win_v;  /* [B][Hkv][C][D] hp_dtype, ring buffer of C = win_cap
                                 rows (C = W when win_cap == 0): position T - W + i
                                 sits in row (win_offset + i) % C */
  int win_offset;             /* 0 <= win_offset < C (0 when W == 0) */
  hq_dtype hp_dtype;          /* dtype of the 16-bit rows: HQ_BF16, HQ_F16 or HQ_F32 */
  int flags;                  /* 0, or HQ_KV_DROP_INT4 */
  int win_cap;                /* 0, or the ring's row count C >= W. With C > W the
                                 ring also keeps the 16-bit rows of the C - W positions
                                 that left the window last, [T - C, T - W) (those
                                 >= 0), which hq_vl_update can promote */
} hq_hybrid_kv;

/* hq_hybrid_kv.flags. HQ_KV_DROP_INT4 leaves the INT4 positions out of the
 * softmax: attention over the VL rows and the window only, the sparse
 * baseline that discards the long tail which the hybrid cache keeps in 4 bits
 * [MR, Improvements and Ablation Studies: Table 12 compares keeping the
 * low-precision long tail with dropping it]. The INT4 planes and the VL
 * bitmap are then not read (they may be null). With k == 0 it is attention
 * over the window alone. */
#define HQ_KV_DROP_INT4 1

/*
 * hq_quantize_kv -- pack rows into INT4 codes plus fp16 scale/zero
 * [AFS, How It Works, item 3: keys and values of the quantized majority are
 * 4-bit; KQ, The abstract: most attention states go to low-bit formats].
 *
 * Source row r of head h (0 <= h < n_heads, 0 <= r < n_rows) starts at
 * element x + h * x_head_stride + r * x_row_stride (x_dtype elements, the D
 * channels contiguous). It is written to row dst_row0 + r of head h in
 * planes with dst_head_rows rows per head:
 *   codes: [n_heads][dst_head_rows] rows in `layout` (TILE16 needs
 *          dst_head_rows % 16 == 0),
 *   sz:    [n_heads][dst_head_rows][D/group][2].
 * Requires dst_row0 + n_rows <= dst_head_rows, D % group == 0, group == 32,
 * D in {64, 128}; x, its row and head strides (in bytes) and codes 16-byte
 * aligned, sz 4-byte aligned. One call covers fewer than 2^31 / 4 groups
 * (n_heads * n_rows * D / 32), else HQ_ERR_UNSUPPORTED: larger planes are
 * quantized in several calls. n_rows == 0 or n_heads == 0 is a no-op.
 */
hq_status hq_quantize_kv(const void *x, hq_dtype x_dtype, int n_heads, int64_t n_rows,
                         int D, int group, int64_t x_head_stride, int64_t x_row_stride,
                         uint8_t *codes, uint16_t *sz, hq_code_layout layout,
                         int64_t dst_head_rows, int64_t dst_row0, void *stream);

/*
 * hq_quantize_kv_pair -- hq_quantize_kv for the keys and the values of the
 * same rows in one launch, in the layouts hq_decode_attn reads: K codes in
 * HQ_LAYOUT_ROWS, V codes in HQ_LAYOUT_TILE16 (same page and section: both
 * keys and values of the quantized majority are 4-bit). This is the per-step
 * eviction of the token that leaves the local window. Arguments as in
 * hq_quantize_kv, with xk/xv sharing dtype and strides; dst_head_rows must be
 * a multiple of 16, and one call covers fewer than 2^31 / 8 groups.
 */
hq_status hq_quantize_kv_pair(const void *xk, const void *xv, hq_dtype x_dtype, int n_heads,
                              int64_t n_rows, int D, int group, int64_t x_head_stride,
                              int64_t x_row_stride, uint8_t *k_codes, uint16_t *k_sz,
                              uint8_t *v_codes, uint16_t *v_sz, int64_t dst_head_rows,
                              int64_t dst_row0, void *stream);

/*
 * hq_gather_rows -- copy the vertical-line rows of K or V into the compact
 * 16-bit buffer [AFS, How It Works, item 1: vertical-line tokens stay in full
 * precision]. For each head h and i < k: dst[h][i][:] = src[h][idx[h][i]][:],
 * src [n_heads][src_rows][D], dst [n_heads][k][D], both of dtype `dtype`,
 * idx [n_heads][k] int32. An index outside [0, src_rows) yields a zero row
 * (nothing outside src is read). k == 0 is a no-op.
 */
hq_status hq_gather_rows(const void *src, hq_dtype dtype, int n_heads, int64_t src_rows, int D,
                         const int32_t *idx, int k, void *dst, void *stream);

/*
 * hq_vl_bitmap -- membership bitmap of the vertical-line set, the form in
 * which the decode kernel skips the INT4 rows of VL positions [AFS, How It
 * Works: the three token sets are disjoint; a VL token is read in 16 bits
 * only]. bits [n_heads][t_cap/32] is overwritten: bit t%32 of word t/32 of
 * head h is set iff t appears in vl_idx[h][0..k). Entries outside [0, t_cap)
 * are ignored. Requires t_cap % 32 == 0.
 */
hq_status hq_vl_bitmap(const int32_t *vl_idx, int n_heads, int k, int64_t t_cap, uint32_t *bits,
                       void *stream);

/*
 * hq_detect_vlines -- vertical-line detector [WPN, body paragraph 4: query
 * vectors are accumulated, one matrix multiplication runs every 64 tokens and
 * its columns are summed; HP: the tokens come from a column-wise attention
 * score and are under 5 %].
 *
 * Accumulate: if q_new != NULL, q_new [B][Hq][D] is copied into slot
 * (step mod R) of the ring q_acc [B][Hq][R][D].
 * Detect: when step mod R == R - 1, or force != 0, for every (b, h) with
 * query heads i in [h*G, (h+1)*G), G = Hq / Hkv:
 *   c_j = sum over r < R and those i of q_acc[b][i][r] . k[b][h][j],
 *   for candidates j in [0, cand_end);
 *   idx_out[b][h] = the k_top positions with the largest c_j, equal scores
 *   to the lower position, in ascending order.
 * k [B][Hkv][k_rows][D] (k_rows >= cand_end). q_new, q_acc and k share
 * `dtype` (HQ_BF16 or HQ_F16; HQ_F32 only with HQ_DETECT_QSUM).
 * score_out (optional) [B][Hkv][cand_end] int64 receives c_j in units of
 * 2^-16 (rounded to nearest even). With HQ_DETECT_MATMUL the product is formed
 * by bf16/fp16 MFMA with fp32 accumulation. The unit's rows are numbered
 * rho = i * R + r (query head i of the group, ring slot r); for each residue
 * rho mod 16 the rows congruent to it are accumulated by the matrix core in
 * fp32, the 16 residue sums of a column are added in fp64 and the total is
 * rounded once to the units. When every input is a multiple of 2^-4 and, for
 * every column j and residue, the sum over its rows and channels of
 * |q[rho][d] k[j][d]| stays below 2^16, every fp32 partial is exact and so
 * are the scores. Otherwise each residue sum carries the fp32 rounding of its
 * accumulation chain: at most 2 n 2^-24 times that absolute sum, n = (G R /
 * 16) D products per residue. With HQ_DETECT_QSUM the query rows are summed in
 * fp64 and multiplied with each key in fp64 (exact for grid inputs within the
 * fp64 range).
 * *ran (host, optional) is set to 1 when detection was enqueued, else 0.
 * Requires 0 <= k_top <= cand_end <= k_rows, 1 <= R <= 1024, D in {64, 128},
 * Hq % Hkv == 0, ws_bytes >= hq_detect_workspace_size(...).
 */
hq_status hq_detect_vlines(const void *q_new, void *q_acc, hq_dtype dtype, int B, int Hq,
                           int Hkv, int D, int R, int64_t step, int force, const void *k,
                           int64_t k_rows, int64_t cand_end, int k_top,
                           hq_detect_method method, int32_t *idx_out, int64_t *score_out,
                           int *ran, void *ws, size_t ws_bytes, void *stream);

/*
 * hq_detect_vlines_cache -- the detector scored from the INT4 key cache
 * instead of the 16-bit keys (a detector variant: the same column scores of
 * summed queries, over the dequantized keys k_hat = c * s + z that the decode
 * already holds, 80 bytes per key at D = 128 instead of 256). Accumulate and
 * cadence exactly as hq_detect_vlines; on detection, for every (b, h):
 *   c_j = (sum over r < R and the group's query heads of q_acc[b][i][r]) .
 *         k_hat[b][h][j], j in [0, cand_end),
 * the query sum and every product and sum in fp64 (exact when the queries
 * are multiples of 2^-4 and the partial sums stay within 2^53 units of their
 * quantum), then top-k as hq_detect_vlines; score_out in units of 2^-16
 * rounded to nearest even. B, Hkv, D, t_cap and the key planes (k_codes in
 * HQ_LAYOUT_ROWS, k_sz) come from kv; cand_end <= min(kv->t_cap, kv->T).
 * Requires ws_bytes >= hq_detect_workspace_size(kv->B, kv->Hkv, cand_end,
 * k_top); errors as hq_detect_vlines, nothing enqueued on error.
 */
hq_status hq_detect_vlines_cache(const void *q_new, void *q_acc, hq_dtype dtype, int Hq, int R,
                                 int64_t step, int force, const hq_hybrid_kv *kv,
                                 int64_t cand_end, int k_top, int32_t *idx_out,
                                 int64_t *score_out, int *ran, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * hq_detect_vlines_mass -- the detector scored by attention mass (a detector
 * variant: the pages measure how much of the attention mass the vertical
 * lines cover [AFS, What to Watch For: about 5 % of the tokens hold 50-85 %
 * of it]). Accumulate and cadence exactly as hq_detect_vlines; on detection,
 * for every (b, h) and every accumulated query row rho of the group:
 *   p_rho,j = softmax over all k_rows keys of sm_scale q_rho . k_j,
 *   c_j = sum over rho of p_rho,j for candidates j in [0, cand_end),
 * then top-k as hq_detect_vlines (ties to the lower position). sm_scale <= 0
 * means 1/sqrt(D). The logits come from bf16/fp16 MFMA with fp32
 * accumulation and the exponentials are fp32, so the scores are
 * approximations of the exact masses (not bit-reproducible against a
 * reference, but deterministic run to run). score_out (optional) receives
 * c_j in int64 units of 2^-22 (so that up to 1024 query rows the score range
 * fits the top-k's 32-bit keys without refinement). Requires dtype HQ_BF16 or HQ_F16, D in {64,
 * 128}, 0 <= k_top <= cand_end <= k_rows, 1 <= R <= 1024, ws_bytes >=
 * hq_detect_mass_workspace_size(B, Hq, Hkv, R, k_rows, cand_end); errors as
 * hq_detect_vlines, nothing enqueued on error.
 */
hq_status hq_detect_vlines_mass(const void *q_new, void *q_acc, hq_dtype dtype, int B, int Hq,
                                int Hkv, int D, int R, int64_t step, int force, const void *k,
                                int64_t k_rows, int64_t cand_end, int k_top, float sm_scale,
                                int32_t *idx_out, int64_t *score_out, int *ran, void *ws,
                                size_t ws_bytes, void *stream);
size_t hq_detect_mass_workspace_size(int B, int Hq, int Hkv, int R, int64_t k_rows,
                                     int64_t cand_end);

size_t hq_detect_workspace_size(int B, int Hkv, int64_t cand_end, int k_top);

/*
 * hq_decode_attn -- one decode step of attention over the hybrid KV cache
 * [AFS, Technical Mechanics, Decode Stage: dequantization fused into the
 * attention computation, decompressing on the fly; KQ, The abstract].
 * For every b and query head i (KV head h = i / G, G = Hq / Hkv):
 *   l_j = sm_scale * q[b][i] . key_j over all positions j in [0, T), key_j the
 *   16-bit row on VL and Win and c * s + z elsewhere; one softmax over all
 *   of them; out[b][i] = sum_j softmax_j * value_j (fp32);
 *   lse[b][i] = log(sum_j exp(l_j)) (natural log, optional).
 * q [B][Hq][D] of q_dtype (HQ_BF16, HQ_F16 or HQ_F32). sm_scale == 0 means
 * 1/sqrt(D). The positions are split into n_splits ranges per (b, h)
 * (0 = automatic, at most 256), each producing a partial softmax state; a
 * second kernel merges them with the log-sum-exp rule in split order.
 * ws: at least hq_decode_workspace_size(kv, Hq, n_splits) bytes (no
 * initialisation needed). Calls that share a workspace and run concurrently
 * on different streams race; calls on one stream do not.
 * Requires Hq % Hkv == 0 and G in {1, 2, 4, 8, 16}; k_sz, v_sz and vl_bits
 * 4-byte aligned, the other buffers 16-byte aligned; with HQ_KV_DROP_INT4,
 * k + W >= 1 (an empty softmax is rejected). With D == 128 and
 * G a multiple of 4, the INT4 keys are dotted with the queries in fp16:
 * bf16 queries must then satisfy |q| < 65504 (magnitudes below 2^-17 round
 * to the fp16 subnormal grid, absolute error below 2^-25).
 */
hq_status hq_decode_attn(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                         float sm_scale, int n_splits, float *out, float *lse, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * hq_decode_step -- hq_decode_attn plus the per-step upkeep of the cache, in
 * the same two kernel launches [AFS, How It Works: a local window of recent
 * tokens stays 16-bit while older tokens are kept in 4 bits; WPN, body
 * paragraph 4: the detector accumulates the decode queries and scores them
 * every 64 tokens]. Same arguments and outputs as hq_decode_attn (out and lse
 * are bitwise the same), and:
 *   q_acc, R, step: if q_acc != NULL, q is copied into slot step % R of the
 *     detector's query ring q_acc [B][Hq][R][D] (q_dtype), exactly as
 *     hq_detect_vlines(q_new = q, ...) would; a following hq_detect_vlines
 *     call then passes q_new = NULL. 1 <= R <= 1024, q_acc 16-byte aligned.
 *   evict: if non-zero and kv->W > 0, the window's oldest row (position
 *     T - W, ring row kv->win_offset of win_k and win_v) is packed into row
 *     T - W of the INT4 planes in the hq_quantize_kv format (K in rows, V in
 *     TILE16, fp16 {s, z}; bit-exact with hq_quantize_kv_pair). This step
 *     reads only INT4 rows [0, T - W), so the row is ready for the next step,
 *     after which the caller advances the window (T + 1, win_offset + 1 mod W)
 *     and writes the new token into the freed ring row. Requires kv->t_cap >=
 *     T - W + 1. The INT4 planes are written through the descriptor's
 *     pointers, which must therefore address writable memory.
 * The upkeep runs in extra workgroups of the merge launch, after every split
 * has read the cache. Errors as hq_decode_attn, plus HQ_ERR_INVALID_ARG for
 * a bad R, step < 0 or a too small t_cap; nothing is enqueued on error.
 */
hq_status hq_decode_step(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                         float sm_scale, int n_splits, float *out, float *lse, void *ws,
                         size_t ws_bytes, void *q_acc, int R, int64_t step, int evict, void *stream);

size_t hq_decode_workspace_size(const hq_hybrid_kv *kv, int Hq, int n_splits);

/*
 * hq_decode_attn_noalloc -- hq_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same arguments,
 * results and errors as hq_decode_attn (bitwise the same outputs for the
 * same inputs and n_splits); the split partials go to a fixed device array
 * of HQ_DECODE_SCRATCH_BYTES inside the library instead of `ws`. It calls
 * no allocation routine. Each GPU it runs on holds its own copy of that
 * array until the process ends; the first call on a device looks up the
 * array's address there. Limits and sharing:
 *  - HQ_ERR_WORKSPACE (nothing enqueued, no device touched) when the split
 *    partials of these sizes would exceed HQ_DECODE_SCRATCH_BYTES, i.e. when
 *    hq_decode_workspace_size(kv, Hq, n_splits) > HQ_DECODE_SCRATCH_BYTES
 *    (16 sequences x 32 query heads at the automatic split count need about
 *    6 MB);
 *  - every call on one GPU shares that GPU's array, and each call overwrites
 *    it before reading it (nothing needs clearing), so calls that overlap in
 *    time on one GPU (different streams, or host threads without ordering)
 *    race; calls on one stream do not.
 */
#define HQ_DECODE_SCRATCH_BYTES (16u << 20)
hq_status hq_decode_attn_noalloc(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                                 float sm_scale, int n_splits, float *out, float *lse, void *stream);

/* The split count hq_decode_attn uses for n_splits == 0. */
int hq_decode_auto_splits(const hq_hybrid_kv *kv, int Hq);

/*
 * hq_vl_update -- apply a re-detection to a rolling hybrid cache, in place
 * [WPN, body paragraph 4: the detector runs every 64 tokens; AFS, How It
 * Works, items 1-2: only the vertical-line tokens and a recent window are kept
 * in 16 bits, the rest in 4 bits]. A decode-time cache holds 16-bit rows only
 * for its VL set and its window ring, so a position can be promoted only
 * while its 16-bit row still exists (a reading of the pages, which say
 * nothing on it). For every (b, h) the candidates are the current VL
 * positions vl_idx[b][h][0..kv->k) (VL row i holds position vl_idx[b][h][i];
 * distinct, all below p0: not checked on the device) and the positions
 * [p0, T - W) that left the window since the last update, whose rows are
 * still in the ring (kv->win_cap > W). The new set is the kv->k candidates
 * with the largest scores[b][h][position] (int64, rows of score_stride >=
 * T - W entries, e.g. the score_out of a detector call over cand_end = T - W),
 * equal scores to the lower position. The VL rows keep their slots: the
 * slot of each dropped position (taken in slot order) receives a promoted
 * one (in position order), so vl_idx, the rows kv->vl_k / kv->vl_v and the
 * bitmap kv->vl_bits are updated through the descriptor's pointers, which
 * must address writable memory; only promoted rows are copied (from the
 * ring). Dropped positions fall back to their INT4 rows, which exist for
 * every position. The ring rows of [p0, T - W) must still hold those
 * positions (each is overwritten C positions later, C = ring rows). The
 * caller passes p0 = T - W at the next update.
 * Requires max(0, T - C) <= p0 <= T - W, T - W - p0 <= 1024 and at most
 * 8192 candidates per head (else HQ_ERR_UNSUPPORTED), D in {64, 128},
 * 16-byte aligned rows (HQ_ERR_INVALID_ARG otherwise). k == 0 or p0 == T - W
 * is a no-op. No workspace; nothing enqueued on error.
 */
hq_status hq_vl_update(const hq_hybrid_kv *kv, int32_t *vl_idx, int64_t p0, const int64_t *scores,
                       int64_t score_stride, void *stream);

/*
 * hq_vl_redetect -- a whole re-detection of a rolling hybrid cache [WPN, body
 * paragraph 4; AFS, How It Works, items 1-2]: the same result as
 * hq_detect_vlines_cache(NULL, q_acc, q_dtype, Hq, R, 0, 1, kv, T - W, 0,
 * NULL, scores, ...) followed by hq_vl_update(kv, vl_idx, p0, scores, T - W),
 * bit for bit where those scores are exact (queries on the 2^-4 grid), but
 * only the candidates are scored: the current VL positions and [p0, T - W),
 * the only positions the update can choose, about k + 64 key rows per head
 * instead of T - W. Per (b, h): the summed query of every ring row of the
 * group's heads (q_acc [B][Hq][R][D], q_dtype == kv->hp_dtype; fp64), each
 * candidate's column score from its INT4 key row (per 32-channel group
 * s sum_e q_e c_e + z sum_e q_e, fp64, rounded once to int64 units of
 * 2^-16), then the update of hq_vl_update. Two launches on `stream`.
 * ws: at least hq_vl_redetect_workspace_size(kv) bytes, 8-byte aligned, no
 * initialisation (the candidates' scores). Requirements and errors as
 * hq_vl_update, plus Hq a multiple of kv->Hkv, 1 <= R <= 1024, the ring and
 * the key codes 16-byte aligned, the scale planes 4-byte aligned
 * (HQ_ERR_INVALID_ARG), HQ_ERR_WORKSPACE for a short workspace. Nothing
 * enqueued on error.
 */
hq_status hq_vl_redetect(const hq_hybrid_kv *kv, int32_t *vl_idx, int64_t p0, const void *q_acc,
                         hq_dtype q_dtype, int Hq, int R, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes hq_vl_redetect needs for this cache: B Hkv (k + 1024)
 * int64 (0 for a null or malformed descriptor). */
size_t hq_vl_redetect_workspace_size(const hq_hybrid_kv *kv);

/*
 * hq_prefill_attn -- causal hybrid-precision prefill attention [AFS, The
 * Technical Mechanics, Prefill Stage: the quantized majority is handled first
 * and the 16-bit vertical lines and local window are overlaid into the
 * result; WPN, summary: queries are quantized as well as keys and values;
 * KQ, The abstract]. For every b, query head qh (KV head h = qh / G) and
 * query position i, over key positions j <= i:
 *   logit(i, j) = sm_scale * q_i . k_j          if j is in vl_idx[b][h] or
 *                                                i - W < j,
 *   logit(i, j) = sm_scale * q_hat_i . k_hat_j  otherwise,
 * q_hat, k_hat being the INT4 round trip of the rows in the hq_quantize_kv
 * format (per token, 32-channel groups, fp16 scale and zero); one causal
 * softmax; out[b][qh][i] = sum_j softmax_j * v_j (fp32), lse[b][qh][i] its
 * natural log-sum-exp (optional).
 * q [B][Hq][T][D], k and v [B][Hkv][T][D], contiguous, of `dtype` (HQ_BF16 or
 * HQ_F16), 16-byte aligned; vl_idx [B][Hkv][k_vl] strictly ascending
 * positions in [0, T) (not checked on the device); out [B][Hq][T][D];
 * sm_scale <= 0 means 1/sqrt(D). Requires D == 128, group == 32,
 * Hq % Hkv == 0. ws: at least hq_prefill_workspace_size bytes, 256-byte
 * aligned, no initialisation needed (it holds the split dequantized Q and K,
 * V and the VL rows in 32-key tiles, and the VL bitmap).
 * Precision: the quantized logits are within about 2^-21 (relative) of the
 * exact q_hat . k_hat; the probabilities are rounded to fp16 for the P . V
 * product and V is converted to fp16 (exact for bf16 magnitudes in
 * [2^-17, 65504]; smaller ones round to the fp16 subnormal grid, absolute
 * error below 2^-25; larger ones are a precondition violation).
 * Errors: HQ_ERR_UNSUPPORTED for another dtype, D or group, T >= 2^23, or
 * more than 5e8 query groups (B * Hq * T * D / 32) in one call; HQ_ERR_INVALID_ARG for
 * sizes < 1, Hq % Hkv != 0, W or k_vl < 0, k_vl > T, null or misaligned
 * pointers; HQ_ERR_WORKSPACE if ws_bytes is too small. Nothing is enqueued
 * on error. The VL positions themselves are not checked on the device.
 */
hq_status hq_prefill_attn(const void *q, const void *k, const void *v, hq_dtype dtype, int B, int Hq,
                          int Hkv, int64_t T, int D, int group, int W, const int32_t *vl_idx, int k_vl,
                          float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * hq_prefill_attn_i8 -- the same operator as hq_prefill_attn, arguments,
 * layouts, workspace and errors alike, with the quantized logits computed in
 * integer form [AFS, The Technical Mechanics, Prefill Stage: the quantized
 * majority runs on low-precision integer arithmetic]: per 32-channel group,
 *   q_hat . k_hat = sq sk C + zk (sq Cq + 32 zq) + zq sk Ck,
 * C the dot product of the two rows' 4-bit codes (an int8 matrix-core
 * product, exact), Cq and Ck the groups' code sums, (s, z) the fp16 scales
 * and zeros. Precision: the main term is sq sk C in fp32 (two roundings);
 * the zero-point terms pass through fp16 hi/lo pairs of
 * (sq Cq + 32 zq) 2^(a - 6), 2^a a power of two per query row that puts the
 * row's largest operand just below 2^14, and of sk Ck / 64 (relative 2^-22;
 * absolute 2^-19 where sk Ck falls below 2^-8); the quantized logits are
 * within about 2^-21 of the sum of the terms' magnitudes. P . V as in
 * hq_prefill_attn. Same speed as hq_prefill_attn on gfx950: the group-scale
 * products per logit load the vector unit as much as the fp16 passes they
 * replace load the matrix cores.
 */
hq_status hq_prefill_attn_i8(const void *q, const void *k, const void *v, hq_dtype dtype, int B, int Hq,
                             int Hkv, int64_t T, int D, int group, int W, const int32_t *vl_idx, int k_vl,
                             float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes,
                             void *stream);

/* Workspace bytes hq_prefill_attn and hq_prefill_attn_i8 need for these
 * sizes (0 if a size is out of range). */
size_t hq_prefill_workspace_size(int B, int Hq, int Hkv, int64_t T, int D, int k_vl);

/*
 * hq_stream_read -- measurement utility (not part of the method): reads
 * `bytes` of device memory at buf once, sequentially, in 16-byte
 * non-temporal loads from 2048 workgroups, and writes nothing in practice
 * (sink is only a guard against the loads being removed: it must hold
 * hq_stream_read_sink_bytes() bytes). Timed over a buffer far larger than
 * the 256 MB Infinity Cache it gives the HBM read ceiling that the decode
 * bandwidth is compared with. buf, bytes 16-byte aligned; HQ_ERR_INVALID_ARG
 * otherwise.
 */
hq_status hq_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
size_t hq_stream_read_sink_bytes(void);

const char *hq_status_string(hq_status s);
const char *hq_last_error(void);
int hq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H_ */
