// Vertical-line detector: query accumulation, Q_acc . K^T every R steps,
// column sums, top-k with lowest-position tie-break.
//
// What is computed: "Hybrid-precision attention reduces compute cost with
// minimal accuracy loss" (wpnews.pro), body paragraph 4 -- the detector
// accumulates query vectors, runs one matrix multiplication every 64 tokens
// and sums the columns; hotpaper.ai paper page, technical-approach list --
// vertical-line tokens are picked from a column-wise attention score and are
// under 5 % of the tokens. The scores are raw logits (a uniform 1/sqrt(D)
// cannot change the ranking) over the R accumulated steps and all G query
// heads of a KV head; the k largest win, equal scores go to the lower position.
//
// Kernels:
//  * acc_kernel      copies this step's queries into the ring slot.
//  * mfma_colsum     (HQ_DETECT_MATMUL) bf16/fp16 MFMA 32x32x16: each wave
//    owns a 32-token column tile with its K fragments in registers and runs
//    over all rows of the unit in 32-row chunks, accumulating every chunk
//    into the same accumulator (so rows congruent mod 32 are summed by the
//    matrix core itself); the 32 row sums of a column are then converted to
//    int64 units of 2^-16 and added exactly.
//  * qsum / gemv     (HQ_DETECT_QSUM) the same scores through linearity:
//    sum the unit's query rows in fp64, then one fp64 dot per key row
//    (HBM-bound: K is read once).
//  * topk_kernel     one workgroup per unit: radix select on a 32-bit
//    order-preserving key (score - min) >> shift, refinement of the boundary
//    bucket on the full int64 score, then an index cut for equal scores and an
//    in-order compaction, so the output is ascending by position.
#include "hq_common.h"

namespace hq {
namespace {

constexpr int64_t kUnitsScale = 65536;   // scores in units of 2^-16

// ---------------------------------------------------------------- accumulate
__global__ __launch_bounds__(256) void acc_kernel(const uint8_t *__restrict__ q_new,
                                                  uint8_t *__restrict__ q_acc, int rows, int row_bytes,
                                                  int R, int slot) {
  const int chunks = row_bytes / 16;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(rows) * chunks) return;
  const int64_t r = gid / chunks;   // b * Hq + i
  const int c = static_cast<int>(gid % chunks);
  const uint4 v = reinterpret_cast<const uint4 *>(q_new + r * row_bytes)[c];
  reinterpret_cast<uint4 *>(q_acc + (r * R + slot) * row_bytes)[c] = v;
}

// ---------------------------------------------------------------- MFMA form
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  if constexpr (DT == HQ_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Grid: units * ceil(cand_end / 128) blocks of 4 waves; wave w of a block owns
// the 32-token column tile 4 * blockIdx_local + w.
template <int D, int DT>
__global__ __launch_bounds__(256) void mfma_colsum_kernel(const uint16_t *__restrict__ q_acc,
                                                          const uint16_t *__restrict__ k, int Hq,
                                                          int Hkv, int R, int64_t k_rows,
                                                          int64_t cand_end, int tiles_per_unit,
                                                          int64_t *__restrict__ scores) {
  constexpr int KC = D / 16;           // k-chunks of 16
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blocks_per_unit = (tiles_per_unit + 3) / 4;
  const int unit = blockIdx.x / blocks_per_unit;             // b * Hkv + h
  const int tile = (blockIdx.x % blocks_per_unit) * 4 + wave;
  if (tile >= tiles_per_unit) return;
  const int G = Hq / Hkv;
  const int b = unit / Hkv;
  const int h = unit % Hkv;
  const int M = G * R;                                        // rows of this unit
  const uint16_t *qrows = q_acc + (static_cast<int64_t>(b) * Hq + h * G) * R * D;
  const int64_t col = static_cast<int64_t>(tile) * 32 + (lane & 31);
  const int half = lane >> 5;

  uint4 bfrag[KC];
  const bool col_ok = col < cand_end;
  const uint16_t *krow = k + (static_cast<int64_t>(unit) * k_rows + (col_ok ? col : 0)) * D;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    bfrag[kc] = col_ok ? *reinterpret_cast<const uint4 *>(krow + kc * 16 + half * 8)
                       : make_uint4(0u, 0u, 0u, 0u);

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int chunks = (M + 31) / 32;
  for (int rc = 0; rc < chunks; ++rc) {
    const int row = rc * 32 + (lane & 31);
    const bool row_ok = row < M;
    const uint16_t *qr = qrows + static_cast<int64_t>(row_ok ? row : 0) * D;
    uint4 afrag[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      afrag[kc] = row_ok ? *reinterpret_cast<const uint4 *>(qr + kc * 16 + half * 8)
                         : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) acc = mfma32<DT>(afrag[kc], bfrag[kc], acc);
  }
  // column = lane & 31; this lane holds 16 of the 32 row residues
  long long s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += __double2ll_rn(static_cast<double>(acc[i]) * 65536.0);
  const long long other = __shfl_xor(s, 32, 64);
  if (half == 0 && col_ok) scores[static_cast<int64_t>(unit) * cand_end + col] = s + other;
}

// ---------------------------------------------------------------- QSUM form
// One block per unit: qs[d] = sum over the unit's rows of q_acc[row][d] in
// fp64, rows split over 8 row phases and combined in fixed order.
template <int DT>
__global__ __launch_bounds__(1024) void qsum_kernel(const void *__restrict__ q_acc, int Hq, int Hkv,
                                                    int R, int D, double *__restrict__ qs) {
  __shared__ double part[8][128];
  const int unit = blockIdx.x;
  const int G = Hq / Hkv;
  const int b = unit / Hkv;
  const int h = unit % Hkv;
  const int M = G * R;
  const int d = threadIdx.x % 128;
  const int ph = threadIdx.x / 128;
  const int64_t base = (static_cast<int64_t>(b) * Hq + h * G) * R * D;
  double s = 0.0;
  if (d < D) {
    for (int r = ph; r < M; r += 8) s += static_cast<double>(load_as_f32<DT>(q_acc, base + static_cast<int64_t>(r) * D + d));
  }
  part[ph][d] = s;
  __syncthreads();
  if (ph == 0 && d < D) {
    double t = 0.0;
#pragma unroll
    for (int p = 0; p < 8; ++p) t += part[p][d];
    qs[static_cast<int64_t>(unit) * D + d] = t;
  }
}

// 256 threads; lanes in groups of D/8 per key row (8 channels per lane).
template <int D, int DT>
__global__ __launch_bounds__(256) void gemv_kernel(const void *__restrict__ k, const double *__restrict__ qs,
                                                   int64_t k_rows, int64_t cand_end, int chunks_per_unit,
                                                   int64_t *__restrict__ scores) {
  constexpr int LPR = D / 8;                // lanes per row
  constexpr int RPB = 256 / LPR;            // rows per block step
  constexpr int CHUNK = 256;                // rows per block
  const int unit = blockIdx.x / chunks_per_unit;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x % chunks_per_unit) * CHUNK;
  const int sub = threadIdx.x % LPR;
  const int rowi = threadIdx.x / LPR;
  double qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[static_cast<int64_t>(unit) * D + sub * 8 + e];
  for (int64_t r = r0 + rowi; r < r0 + CHUNK; r += RPB) {
    const bool ok = r < cand_end;
    double acc = 0.0;
    if (ok) {
      const int64_t off = (static_cast<int64_t>(unit) * k_rows + r) * D + sub * 8;
      if constexpr (DT == HQ_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(k) + off);
        const float4 a = p[0], c = p[1];
        const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fma(qv[e], static_cast<double>(v[e]), acc);
      } else {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(k) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float lo, hi;
          if constexpr (DT == HQ_BF16) {
            lo = bf16_to_f32(w[e] & 0xFFFFu);
            hi = bf16_to_f32(w[e] >> 16);
          } else {
            lo = f16_to_f32(w[e] & 0xFFFFu);
            hi = f16_to_f32(w[e] >> 16);
          }
          acc = fma(qv[2 * e], static_cast<double>(lo), acc);
          acc = fma(qv[2 * e + 1], static_cast<double>(hi), acc);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (ok && sub == 0)
      scores[static_cast<int64_t>(unit) * cand_end + r] = __double2ll_rn(acc * 65536.0);
  }
}

// ---------------------------------------------------------------- top-k
constexpr int kTopkThreads = 1024;

__device__ __forceinline__ unsigned long long block_reduce_min_max(long long v_min, long long v_max,
                                                                   long long *sh, long long *out_min,
                                                                   long long *out_max) {
  // sh: 2 * 32 entries
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const long long a = __shfl_xor(v_min, m, 64);
    const long long c = __shfl_xor(v_max, m, 64);
    v_min = a < v_min ? a : v_min;
    v_max = c > v_max ? c : v_max;
  }
  if (lane == 0) { sh[w] = v_min; sh[32 + w] = v_max; }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long mn = sh[0], mx = sh[32];
    for (int i = 1; i < kTopkThreads / 64; ++i) {
      mn = sh[i] < mn ? sh[i] : mn;
      mx = sh[32 + i] > mx ? sh[32 + i] : mx;
    }
    *out_min = mn;
    *out_max = mx;
  }
  __syncthreads();
  return 0;
}

// exclusive scan of one int per thread over the block; returns the prefix
// and writes the total to *total
__device__ __forceinline__ int block_exclusive_scan(int v, int *sh, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int t = __shfl_up(inc, m, 64);
    if (lane >= m) inc += t;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kTopkThreads / 64; ++i) {
      const int t = sh[i];
      sh[i] = run;
      run += t;
    }
    sh[kTopkThreads / 64] = run;
  }
  __syncthreads();
  const int pre = sh[w] + inc - v;
  *total = sh[kTopkThreads / 64];
  __syncthreads();
  return pre;
}

// Radix select over the 32-bit keys of the selected elements: finds the key
// value kappa of the k_rem-th largest and how many with key == kappa to take.
// key_of(j) returns (valid, key).
template <typename KeyFn>
__device__ void radix_select32(int64_t n, int k_rem, KeyFn key_of, unsigned *hist, int *sh_i,
                               unsigned *kappa_out, int *take_out) {
  unsigned prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t j = threadIdx.x; j < n; j += kTopkThreads) {
      unsigned key;
      if (key_of(j, &key) && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, d = 255;
      for (; d > 0; --d) {
        if (cum + static_cast<int>(hist[d]) >= k_rem) break;
        cum += hist[d];
      }
      sh_i[0] = d;
      sh_i[1] = k_rem - cum;
    }
    __syncthreads();
    prefix |= static_cast<unsigned>(sh_i[0]) << shift;
    pmask |= 255u << shift;
    k_rem = sh_i[1];
    __syncthreads();
  }
  *kappa_out = prefix;
  *take_out = k_rem;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const int64_t *__restrict__ scores,
                                                            int64_t n, int k_top,
                                                            int32_t *__restrict__ idx_out) {
  __shared__ unsigned hist[256];
  __shared__ long long shl[64];
  __shared__ int shi[kTopkThreads / 64 + 2];
  __shared__ long long s_min, s_max;
  __shared__ unsigned s_kappa;
  __shared__ int s_take;
  const int unit = blockIdx.x;
  const int64_t *sc = scores + static_cast<int64_t>(unit) * n;
  int32_t *out = idx_out + static_cast<int64_t>(unit) * k_top;
  if (k_top == 0) return;

  // 1. min / max of the scores
  long long mn = 0x7FFFFFFFFFFFFFFFLL, mx = -0x7FFFFFFFFFFFFFFFLL - 1;
  for (int64_t j = threadIdx.x; j < n; j += kTopkThreads) {
    const long long v = sc[j];
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
  }
  block_reduce_min_max(mn, mx, shl, &s_min, &s_max);
  const long long smin = s_min;
  const unsigned long long range = static_cast<unsigned long long>(s_max) - static_cast<unsigned long long>(smin);
  const int bits = range == 0 ? 0 : 64 - __clzll(static_cast<long long>(range));
  const int shift = bits > 32 ? bits - 32 : 0;

  // 2. radix select on key = (score - min) >> shift
  auto key32 = [&](int64_t j, unsigned *key) -> bool {
    *key = static_cast<unsigned>((static_cast<unsigned long long>(sc[j]) - static_cast<unsigned long long>(smin)) >> shift);
    return true;
  };
  radix_select32(n, k_top, key32, hist, shi, &s_kappa, &s_take);
  const unsigned kappa = s_kappa;
  int take = s_take;

  // 3. refine the boundary bucket on the low `shift` bits of the score
  unsigned long long tau = (static_cast<unsigned long long>(kappa) << shift);   // score - min
  if (shift > 0) {
    auto key_lo = [&](int64_t j, unsigned *key) -> bool {
      const unsigned long long v = static_cast<unsigned long long>(sc[j]) - static_cast<unsigned long long>(smin);
      *key = static_cast<unsigned>(v & ((1ull << shift) - 1ull));
      return static_cast<unsigned>(v >> shift) == kappa;
    };
    radix_select32(n, take, key_lo, hist, shi, &s_kappa, &s_take);
    tau |= s_kappa;
    take = s_take;
  }
  const long long tau_s = static_cast<long long>(tau + static_cast<unsigned long long>(smin));

  // 4. among scores == tau_s take the `take` lowest positions; then compact
  const int64_t per = (n + kTopkThreads - 1) / kTopkThreads;
  const int64_t j0 = threadIdx.x * per;
  const int64_t j1 = (j0 + per) < n ? (j0 + per) : n;
  int eq = 0, gt = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const long long v = sc[j];
    eq += (v == tau_s);
    gt += (v > tau_s);
  }
  int tot;
  int eq_before = block_exclusive_scan(eq, shi, &tot);
  // selected in this segment: all gt, and eq ones whose global rank < take
  int sel = gt;
  {
    int r = eq_before;
    for (int64_t j = j0; j < j1; ++j)
      if (sc[j] == tau_s) { sel += (r < take); ++r; }
  }
  int pos = block_exclusive_scan(sel, shi, &tot);
  {
    int r = eq_before;
    for (int64_t j = j0; j < j1; ++j) {
      const long long v = sc[j];
      bool s = v > tau_s;
      if (v == tau_s) { s = r < take; ++r; }
      if (s && pos < k_top) out[pos++] = static_cast<int32_t>(j);
    }
  }
}

// ---------------------------------------------------------------- workspace
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
struct DetWs {
  size_t scores, qs, total;
};
DetWs det_ws(int B, int Hkv, int64_t cand_end) {
  DetWs L{};
  L.scores = 0;
  L.qs = align_up(static_cast<size_t>(B) * Hkv * cand_end * sizeof(int64_t), 256);
  L.total = L.qs + static_cast<size_t>(B) * Hkv * 128 * sizeof(double);
  return L;
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" size_t hq_detect_workspace_size(int B, int Hkv, int64_t cand_end, int k_top) {
  (void)k_top;
  if (B < 1 || Hkv < 1 || cand_end < 0) return 0;
  return det_ws(B, Hkv, cand_end).total;
}

extern "C" hq_status hq_detect_vlines(const void *q_new, void *q_acc, hq_dtype dtype, int B, int Hq,
                                      int Hkv, int D, int R, int64_t step, int force, const void *k,
                                      int64_t k_rows, int64_t cand_end, int k_top,
                                      hq_detect_method method, int32_t *idx_out, int64_t *score_out,
                                      int *ran, void *ws, size_t ws_bytes, void *stream) {
  if (ran) *ran = 0;
  if (!dtype_ok(dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: bad dtype");
  if (method != HQ_DETECT_MATMUL && method != HQ_DETECT_QSUM)
    return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: bad method");
  if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: bad head counts");
  if (D != 64 && D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines: D must be 64 or 128");
  if (R < 1 || R > 1024) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: need 1 <= R <= 1024");
  if (step < 0) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: step < 0");
  if (k_top < 0 || cand_end < k_top || k_rows < cand_end)
    return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: need 0 <= k_top <= cand_end <= k_rows");
  if (cand_end > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines: cand_end too large");
  if (dtype == HQ_F32 && method == HQ_DETECT_MATMUL)
    return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines: fp32 inputs need HQ_DETECT_QSUM");
  if (!q_acc) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: null q_acc");
  const int eb = dtype_bytes(dtype);
  const int slot = static_cast<int>(step % R);
  hipStream_t st = as_stream(stream);
  const bool detect = force || slot == R - 1;
  if (detect) {
    if (!k || (k_top > 0 && !idx_out)) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: null k or idx_out");
    const DetWs L = det_ws(B, Hkv, cand_end);
    const bool need_ws_scores = (score_out == nullptr);
    const size_t need = need_ws_scores || method == HQ_DETECT_QSUM ? L.total : 0;
    if (need > 0 && (!ws || ws_bytes < need))
      return fail(HQ_ERR_WORKSPACE, "hq_detect_vlines: workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(q_acc) % 16)
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: k and q_acc must be 16-byte aligned");
  }
  if (q_new) {
    if (reinterpret_cast<uintptr_t>(q_new) % 16) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines: q_new must be 16-byte aligned");
    const int rows = B * Hq;
    const int row_bytes = D * eb;
    const int64_t threads = static_cast<int64_t>(rows) * (row_bytes / 16);
    hipLaunchKernelGGL(acc_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint8_t *>(q_new), static_cast<uint8_t *>(q_acc), rows, row_bytes, R,
                       slot);
    hq_status s = check_launch("hq_detect_vlines (accumulate)");
    if (s != HQ_OK) return s;
  }
  if (!detect) { clear_error(); return HQ_OK; }
  const DetWs L = det_ws(B, Hkv, cand_end);
  int64_t *scores = score_out ? score_out : reinterpret_cast<int64_t *>(static_cast<uint8_t *>(ws) + L.scores);
  const int units = B * Hkv;
  if (cand_end > 0) {
    if (method == HQ_DETECT_MATMUL) {
      const int tiles = static_cast<int>((cand_end + 31) / 32);
      const int blocks = units * ((tiles + 3) / 4);
      const uint16_t *qa = static_cast<const uint16_t *>(q_acc);
      const uint16_t *kk = static_cast<const uint16_t *>(k);
      if (D == 128) {
        if (dtype == HQ_BF16)
          hipLaunchKernelGGL((mfma_colsum_kernel<128, HQ_BF16>), dim3(blocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, tiles, scores);
        else
          hipLaunchKernelGGL((mfma_colsum_kernel<128, HQ_F16>), dim3(blocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, tiles, scores);
      } else {
        if (dtype == HQ_BF16)
          hipLaunchKernelGGL((mfma_colsum_kernel<64, HQ_BF16>), dim3(blocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, tiles, scores);
        else
          hipLaunchKernelGGL((mfma_colsum_kernel<64, HQ_F16>), dim3(blocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, tiles, scores);
      }
    } else {
      double *qs = reinterpret_cast<double *>(static_cast<uint8_t *>(ws) + L.qs);
      switch (dtype) {
        case HQ_F32: hipLaunchKernelGGL(qsum_kernel<HQ_F32>, dim3(units), dim3(1024), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
        case HQ_BF16: hipLaunchKernelGGL(qsum_kernel<HQ_BF16>, dim3(units), dim3(1024), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
        default: hipLaunchKernelGGL(qsum_kernel<HQ_F16>, dim3(units), dim3(1024), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
      }
      const int cpu = static_cast<int>((cand_end + 255) / 256);
      const dim3 grid(static_cast<unsigned>(units * cpu));
#define HQ_GEMV(DD, TT) hipLaunchKernelGGL((gemv_kernel<DD, TT>), grid, dim3(256), 0, st, k, qs, k_rows, cand_end, cpu, scores)
      if (D == 128) {
        if (dtype == HQ_F32) HQ_GEMV(128, HQ_F32); else if (dtype == HQ_BF16) HQ_GEMV(128, HQ_BF16); else HQ_GEMV(128, HQ_F16);
      } else {
        if (dtype == HQ_F32) HQ_GEMV(64, HQ_F32); else if (dtype == HQ_BF16) HQ_GEMV(64, HQ_BF16); else HQ_GEMV(64, HQ_F16);
      }
#undef HQ_GEMV
    }
    hq_status s = check_launch("hq_detect_vlines (scores)");
    if (s != HQ_OK) return s;
  }
  if (k_top > 0) {
    hipLaunchKernelGGL(topk_kernel, dim3(units), dim3(kTopkThreads), 0, st, scores, cand_end, k_top, idx_out);
    hq_status s = check_launch("hq_detect_vlines (top-k)");
    if (s != HQ_OK) return s;
  }
  if (ran) *ran = 1;
  clear_error();
  return HQ_OK;
}
