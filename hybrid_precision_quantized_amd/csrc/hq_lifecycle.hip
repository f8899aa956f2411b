// Re-detection of the vertical-line set in a rolling hybrid cache.
//
// What is computed: "Hybrid-precision attention reduces compute cost with
// minimal accuracy loss" (wpnews.pro), body paragraph 4 -- the detector
// runs every 64 tokens over the accumulated queries; "HyQuant ... Explained
// for Beginners" (aifromscratch.in), "How It Works", items 1-2 -- only the
// vertical-line tokens and a recent window stay 16-bit, everything older is
// 4-bit. A decode-time cache therefore holds 16-bit rows only for the current
// VL set and for the window ring; a ring with more rows than the window also
// keeps the rows of the positions that left the window since the last
// detection. A new detection can promote a position only while its 16-bit
// row exists: the candidates are the current VL set and those recent
// positions, and the new set is the k best of them by the detector's score
// (equal scores to the lower position). Dropped VL positions fall back to
// their INT4 rows, which exist for every position.
//
// Kernel: one workgroup of 1024 threads per (sequence, KV head).
//  * The n <= 8192 candidates (old VL list, then the recent range: ascending
//    positions, since every old VL position precedes the range) are loaded
//    with their scores as order-preserving 64-bit keys and sorted in LDS by a
//    bitonic network, best first (larger key, then lower candidate index =
//    lower position); padding entries sort last.
//  * The first k_new sorted entries are flagged; a block scan over the
//    candidates in order gives each selected one its output slot, so the new
//    list comes out ascending.
//  * All threads then copy the selected 16-bit K and V rows (from the old VL
//    rows or from the ring) into the new buffers in 16-byte pieces, and the
//    VL bitmap words are updated with integer atomics (bits of dropped VL
//    positions cleared, bits of promoted ring positions set).
#include "hq_common.h"

namespace hq {
namespace {

constexpr int kUpdThreads = 1024;
constexpr int kMaxCand = 8192;

struct UpdParams {
  const int32_t *old_idx;        // [units][k_old]
  const int64_t *scores;         // [units][stride]
  const uint8_t *old_k, *old_v;  // [units][k_old][row_bytes]
  const uint8_t *ring_k, *ring_v;// [units][C][row_bytes]
  int32_t *new_idx;              // [units][k_new]
  uint8_t *new_k, *new_v;        // [units][k_new][row_bytes]
  uint32_t *bits;                // [units][words]
  int64_t stride, words, p0, nq; // nq = T - W
  int k_old, k_new, C, win_offset, row_bytes;
};

__device__ __forceinline__ unsigned long long order_key(long long v) {
  return static_cast<unsigned long long>(v) ^ 0x8000000000000000ull;
}

__global__ __launch_bounds__(kUpdThreads) void vl_update_kernel(UpdParams P) {
  __shared__ unsigned long long key[kMaxCand];
  __shared__ uint16_t id[kMaxCand];
  __shared__ uint16_t src_of[kMaxCand];     // output slot -> candidate index
  __shared__ uint8_t taken[kMaxCand];
  __shared__ int scan[kUpdThreads];
  const int64_t unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_old = P.k_old;
  const int n = n_old + static_cast<int>(P.nq - P.p0);
  int npow = 2;
  while (npow < n) npow <<= 1;
  const int32_t *oi = P.old_idx + unit * n_old;
  auto cand_pos = [&](int i) -> int64_t {
    return i < n_old ? static_cast<int64_t>(oi[i]) : P.p0 + (i - n_old);
  };

  // ---- candidates and their keys
  for (int i = tid; i < npow; i += kUpdThreads) {
    if (i < n) {
      key[i] = order_key(P.scores[unit * P.stride + cand_pos(i)]);
      id[i] = static_cast<uint16_t>(i);
    } else {
      key[i] = 0ull;
      id[i] = 0xFFFFu;
    }
    taken[i] = 0;
  }
  __syncthreads();

  // ---- bitonic sort, best first: larger key, then lower candidate index
  auto better = [&](int a, int b) {
    const unsigned long long ka = key[a], kb = key[b];
    return ka != kb ? ka > kb : id[a] < id[b];
  };
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (npow >> 1); i += kUpdThreads) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        if (up ? better(hi, lo) : better(lo, hi)) {
          const unsigned long long tk = key[lo];
          key[lo] = key[hi];
          key[hi] = tk;
          const uint16_t ti = id[lo];
          id[lo] = id[hi];
          id[hi] = ti;
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < P.k_new; r += kUpdThreads) taken[id[r]] = 1;
  __syncthreads();

  // ---- output slots in candidate (= position) order: block exclusive scan
  constexpr int kPer = kMaxCand / kUpdThreads;               // candidates per thread
  const int c0 = tid * kPer;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) cnt += (c0 + e < n) ? taken[c0 + e] : 0;
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kUpdThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int slot = scan[tid] - cnt;
  const int64_t wbase = unit * P.words;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = c0 + e;
    if (i >= n) break;
    const int64_t pos = cand_pos(i);
    const uint32_t bit = 1u << (pos & 31);
    if (taken[i]) {
      src_of[slot] = static_cast<uint16_t>(i);
      P.new_idx[unit * P.k_new + slot] = static_cast<int32_t>(pos);
      ++slot;
      if (i >= n_old) atomicOr(&P.bits[wbase + (pos >> 5)], bit);         // promoted from the ring
    } else if (i < n_old) {
      atomicAnd(&P.bits[wbase + (pos >> 5)], ~bit);                      // demoted to its INT4 row
    }
  }
  __syncthreads();

  // ---- the selected 16-bit rows, 16 bytes per thread and step
  const int pieces = P.row_bytes / 16;
  const int64_t total = static_cast<int64_t>(P.k_new) * pieces;
  for (int64_t e = tid; e < total; e += kUpdThreads) {
    const int r = static_cast<int>(e / pieces);
    const int c = static_cast<int>(e % pieces);
    const int i = src_of[r];
    const uint8_t *sk, *sv;
    if (i < n_old) {
      const int64_t off = (unit * n_old + i) * P.row_bytes;
      sk = P.old_k + off;
      sv = P.old_v + off;
    } else {
      // position p0 + (i - n_old) = T - W + j with j < 0 sits in ring row (win_offset + j) mod C
      const int64_t j = P.p0 + (i - n_old) - P.nq;
      const int64_t ring = (P.win_offset + j + P.C) % P.C;
      const int64_t off = (unit * P.C + ring) * P.row_bytes;
      sk = P.ring_k + off;
      sv = P.ring_v + off;
    }
    const int64_t doff = (unit * P.k_new + r) * P.row_bytes + 16 * c;
    *reinterpret_cast<uint4 *>(P.new_k + doff) = *reinterpret_cast<const uint4 *>(sk + 16 * c);
    *reinterpret_cast<uint4 *>(P.new_v + doff) = *reinterpret_cast<const uint4 *>(sv + 16 * c);
  }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" hq_status hq_vl_update(const hq_hybrid_kv *kv, const int32_t *vl_idx, int64_t p0,
                                  const int64_t *scores, int64_t score_stride, int k_new, int32_t *new_idx,
                                  void *new_vl_k, void *new_vl_v, uint32_t *vl_bits, void *stream) {
  if (!kv) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: null descriptor");
  if (kv->B < 1 || kv->Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: B, Hkv must be >= 1");
  if (kv->D != 64 && kv->D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_vl_update: D must be 64 or 128");
  if (!dtype_ok(kv->hp_dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: bad dtype");
  if (kv->T < 1 || kv->W < 0 || kv->W > kv->T || kv->k < 0 || kv->k > kv->T - kv->W)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: need 0 <= W <= T and 0 <= k <= T - W");
  const int64_t C = kv->win_cap > 0 ? kv->win_cap : kv->W;
  if (C < kv->W) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: win_cap must be 0 or >= W");
  if (kv->W > 0 && (kv->win_offset < 0 || kv->win_offset >= C))
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: win_offset out of range");
  const int64_t nq = kv->T - kv->W;
  if (p0 > nq || p0 < 0 || p0 < kv->T - C)
    return fail(HQ_ERR_INVALID_ARG,
                "hq_vl_update: p0 = %lld must lie in [max(0, T - win_cap), T - W] = [%lld, %lld]: only "
                "positions whose 16-bit rows are still in the ring can be promoted",
                static_cast<long long>(p0), static_cast<long long>(kv->T - C > 0 ? kv->T - C : 0),
                static_cast<long long>(nq));
  const int64_t n = kv->k + (nq - p0);
  if (k_new < 0 || k_new > n)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: need 0 <= k_new <= k + (T - W - p0) = %lld",
                static_cast<long long>(n));
  if (n > kMaxCand)
    return fail(HQ_ERR_UNSUPPORTED, "hq_vl_update: %lld candidates per head exceed %d", static_cast<long long>(n),
                kMaxCand);
  if (kv->t_cap < nq || kv->t_cap % 32 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: t_cap must be >= T - W and a multiple of 32");
  if (score_stride < nq) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: score_stride < T - W");
  if (n == 0) { clear_error(); return HQ_OK; }
  const int64_t units = static_cast<int64_t>(kv->B) * kv->Hkv;
  const int row_bytes = kv->D * dtype_bytes(kv->hp_dtype);
  if (!scores || !vl_bits || (kv->k > 0 && (!vl_idx || !kv->vl_k || !kv->vl_v)) ||
      (nq > p0 && (!kv->win_k || !kv->win_v)) || (k_new > 0 && (!new_idx || !new_vl_k || !new_vl_v)))
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: null pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(kv->vl_k) | reinterpret_cast<uintptr_t>(kv->vl_v) |
                       reinterpret_cast<uintptr_t>(kv->win_k) | reinterpret_cast<uintptr_t>(kv->win_v) |
                       reinterpret_cast<uintptr_t>(new_vl_k) | reinterpret_cast<uintptr_t>(new_vl_v);
  if (al % 16 || reinterpret_cast<uintptr_t>(vl_bits) % 4 || reinterpret_cast<uintptr_t>(scores) % 8 ||
      reinterpret_cast<uintptr_t>(vl_idx) % 4 || reinterpret_cast<uintptr_t>(new_idx) % 4)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: misaligned buffer (rows 16 bytes, words 4, scores 8)");
  const size_t old_rows = static_cast<size_t>(units) * kv->k * row_bytes;
  const size_t new_rows = static_cast<size_t>(units) * k_new * row_bytes;
  const size_t ring_rows = static_cast<size_t>(units) * C * row_bytes;
  if (overlaps(new_vl_k, new_rows, kv->vl_k, old_rows) || overlaps(new_vl_k, new_rows, kv->vl_v, old_rows) ||
      overlaps(new_vl_v, new_rows, kv->vl_k, old_rows) || overlaps(new_vl_v, new_rows, kv->vl_v, old_rows) ||
      overlaps(new_vl_k, new_rows, kv->win_k, ring_rows) || overlaps(new_vl_v, new_rows, kv->win_v, ring_rows) ||
      overlaps(new_vl_k, new_rows, new_vl_v, new_rows) ||
      overlaps(new_idx, static_cast<size_t>(units) * k_new * 4, vl_idx, static_cast<size_t>(units) * kv->k * 4))
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: the new VL buffers must not overlap the old ones or the ring");
  if (units > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_vl_update: too many heads");
  UpdParams P{};
  P.old_idx = vl_idx;
  P.scores = scores;
  P.old_k = static_cast<const uint8_t *>(kv->vl_k);
  P.old_v = static_cast<const uint8_t *>(kv->vl_v);
  P.ring_k = static_cast<const uint8_t *>(kv->win_k);
  P.ring_v = static_cast<const uint8_t *>(kv->win_v);
  P.new_idx = new_idx;
  P.new_k = static_cast<uint8_t *>(new_vl_k);
  P.new_v = static_cast<uint8_t *>(new_vl_v);
  P.bits = vl_bits;
  P.stride = score_stride;
  P.words = kv->t_cap / 32;
  P.p0 = p0;
  P.nq = nq;
  P.k_old = kv->k;
  P.k_new = k_new;
  P.C = static_cast<int>(C);
  P.win_offset = kv->win_offset;
  P.row_bytes = row_bytes;
  hipLaunchKernelGGL(vl_update_kernel, dim3(static_cast<unsigned>(units)), dim3(kUpdThreads), 0,
                     as_stream(stream), P);
  return check_launch("hq_vl_update");
}
