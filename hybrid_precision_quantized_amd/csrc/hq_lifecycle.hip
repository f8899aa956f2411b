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
// Kernel: one workgroup of 1024 threads per (sequence, KV head), in place.
//  * The n <= 8192 candidates (the current VL rows in slot order, then the
//    recent range) are loaded into LDS with their scores as order-preserving
//    64-bit keys. The k best (larger score, then lower position) are found
//    by a radix select over the rank key (score key minus the smallest, then
//    the inverted position: B + 32 bits, B the width of the score range),
//    most significant 12 bits first: per pass a 4096-bin histogram of the
//    candidates still tied with the threshold, one wave's scan for the digit
//    where the count from the top reaches what is still needed, and the
//    candidates above it taken. With 4096 bins over the score range the
//    boundary bin usually holds a few candidates, and once at most 64 are
//    left one wave ranks them directly: one pass in the common case, a few
//    for heavy ties.
//  * The VL rows keep their slots: the slot of every dropped VL position is
//    refilled with a promoted one (the j-th freed slot in slot order takes
//    the j-th promoted position in position order, both found with one
//    block scan), so only the promoted rows are copied, from the ring, and
//    only their index entries change. The VL bitmap words are updated with
//    integer atomics (bits of dropped positions cleared, of promoted ones
//    set). The rows are a set for the attention: their order is irrelevant
//    to it, and the slot rule makes it deterministic.
//  * hq_vl_redetect scores only the candidates, the only positions the
//    update can choose (about k + 64 key rows per head instead of all
//    T - W), in a kernel of its own with many workgroups per head: each sums
//    the unit's query ring (fp64, in LDS) and scores 256 candidates per round
//    (D = 128; 512 at D = 64; up to 8 rounds) from their INT4 key rows, in the INT4-key GEMV's
//    arithmetic (per 32-channel group s sum_e q_e c_e + z sum_e q_e in fp64,
//    the groups added by butterfly, rounded once to units of 2^-16), into a
//    workspace indexed by candidate; the update kernel then reads them by
//    candidate instead of by position. Scoring in the single update
//    workgroup of each head made that workgroup's vector unit the bound.
#include "hq_common.h"

namespace hq {
namespace {

constexpr int kUpdThreads = 1024;
constexpr int kMaxCand = 8192;
constexpr int kMaxMoved = 1024;   // positions that may leave the window between two updates

struct UpdParams {
  int32_t *idx;                  // [units][k] in/out: position of each VL slot
  const int64_t *scores;         // [units][stride], by position, or by candidate when by_cand
  int64_t *cand_scores;          // scoring kernel: out [units][k + nq - p0]
  const void *q_acc;             // scoring kernel: query ring [B][Hq][R][D]
  const uint8_t *k_codes;        //   INT4 key rows [units][t_cap][D / 2]
  const uint32_t *k_sz;          //   fp16 {s, z} words [units][t_cap][D / 32]
  int64_t t_cap;
  int Hq, Hkv, R, by_cand;
  uint8_t *vl_k, *vl_v;          // [units][k][row_bytes] in/out
  const uint8_t *ring_k, *ring_v;// [units][C][row_bytes]
  uint32_t *bits;                // [units][words]
  int64_t stride, words, p0, nq; // nq = T - W
  int k, C, win_offset, row_bytes;
};

constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ unsigned long long order_key(long long v) {
  return static_cast<unsigned long long>(v) ^ 0x8000000000000000ull;
}

// Bits [sh, sh + w) (w <= 12) of a candidate's rank key R = hi 2^32 + lo:
// hi = its score key minus the smallest (fewer than 64 bits), lo = 2^32 - 1 -
// position (a lower position ranks higher). Keys are distinct because
// positions are.
__device__ __forceinline__ uint32_t rank_bits(unsigned long long hi, int32_t pos, int sh, int w) {
  const uint32_t lo = 0xFFFFFFFFu - static_cast<uint32_t>(pos);
  const uint32_t mask = (1u << w) - 1u;
  if (sh >= 32) return static_cast<uint32_t>(hi >> (sh - 32)) & mask;
  if (sh + w <= 32) return (lo >> sh) & mask;
  return static_cast<uint32_t>((static_cast<unsigned long long>(lo) >> sh) | (hi << (32 - sh))) & mask;
}

template <int DT>
__device__ __forceinline__ float ring_half(uint32_t h) {
  if constexpr (DT == HQ_BF16) return bf16_to_f32(h);
  else return f16_to_f32(h);
}

// Candidate scores of a re-detection: block (unit, c) scores candidates
// [c RPB CPR, (c + 1) RPB CPR) of the unit (the VL list, then [p0, T - W)),
// CPR per round, RPB = rounds rounds (<= kMaxRounds; more rounds per block
// when there are many heads, so that fewer blocks read each query ring).
// Lane (candidate, 32-channel group g) reads the candidate's position and
// issues the loads of its key codes and {s, z} word for every round first;
// then the block sums the unit's query ring (thread (row group, 8-channel
// slice) adds its rows, the lanes of a wave sharing a slice combine by
// butterfly, the waves' sums meet in LDS in wave order), and each lane adds
// its group terms.
constexpr int kMaxRounds = 8;
template <int DT, int D>
__global__ __launch_bounds__(kUpdThreads) void redetect_scores_kernel(UpdParams P, int rounds) {
  constexpr int NG = D / 32, CPR = kUpdThreads / NG;     // candidates per round
  __shared__ double part[kUpdThreads / 64][D];
  __shared__ double qsh[D];
  const int k = P.k;
  const int n = k + static_cast<int>(P.nq - P.p0);
  const int cpb = CPR * rounds;
  const int nb = (n + cpb - 1) / cpb;
  const int64_t unit = blockIdx.x / nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = tid % NG;
  const int i0 = static_cast<int>(blockIdx.x % nb) * cpb + tid / NG;
  uint4 cw[kMaxRounds];
  uint32_t cz[kMaxRounds];
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    const int i = i0 + CPR * r;
    cw[r] = make_uint4(0u, 0u, 0u, 0u);
    cz[r] = 0u;
    if (r < rounds && i < n) {
      const int32_t p = i < k ? P.idx[unit * k + i] : static_cast<int32_t>(P.p0 + (i - k));
      const int64_t row = unit * P.t_cap + p;
      cw[r] = *reinterpret_cast<const uint4 *>(P.k_codes + row * (D / 2) + g * 16);
      cz[r] = P.k_sz[row * NG + g];
    }
  }
  {
    constexpr int LPR = D / 8, RG = kUpdThreads / LPR;
    constexpr int kRing = DT == HQ_F32 ? 4 : 8;
    const int G = P.Hq / P.Hkv;
    const int M = G * P.R;
    const int64_t b = unit / P.Hkv, h = unit % P.Hkv;
    const int sub = tid % LPR, rg = tid / LPR;
    const int64_t base = (b * P.Hq + h * G) * P.R * D + sub * 8;
    double sq[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int r0 = rg; r0 < M; r0 += RG * kRing) {
      if constexpr (DT == HQ_F32) {
        float4 x[kRing][2];
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const int r = r0 + RG * j;
          if (r < M) {
            const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(P.q_acc) + base +
                                                               static_cast<int64_t>(r) * D);
            x[j][0] = q[0];
            x[j][1] = q[1];
          }
        }
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          if (r0 + RG * j < M) {
            const float v[8] = {x[j][0].x, x[j][0].y, x[j][0].z, x[j][0].w, x[j][1].x, x[j][1].y, x[j][1].z, x[j][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sq[e] += static_cast<double>(v[e]);
          }
        }
      } else {
        uint4 u[kRing];
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const int r = r0 + RG * j;
          if (r < M)
            u[j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(P.q_acc) + base +
                                                    static_cast<int64_t>(r) * D);
        }
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          if (r0 + RG * j < M) {
            const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sq[2 * e] += static_cast<double>(ring_half<DT>(w[e] & 0xFFFFu));
              sq[2 * e + 1] += static_cast<double>(ring_half<DT>(w[e] >> 16));
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) sq[e] += __shfl_xor(sq[e], m, 64);
    if (lane < LPR)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[tid >> 6][sub * 8 + e] = sq[e];
    __syncthreads();
    if (tid < D) {
      double t = 0.0;
      for (int w = 0; w < kUpdThreads / 64; ++w) t += part[w][tid];
      qsh[tid] = t;
    }
    __syncthreads();
  }
  double qv[32];
  double qsum = 0.0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    qv[e] = qsh[g * 32 + e];
    qsum += qv[e];
  }
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    if (r >= rounds) break;                 // uniform
    const int i = i0 + CPR * r;
    const uint32_t word[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc = fma(qv[e], static_cast<double>((word[e >> 3] >> (4 * (e & 7))) & 0xFu), acc);
    const double sc = static_cast<double>(f16_to_f32(cz[r] & 0xFFFFu));
    const double z = static_cast<double>(f16_to_f32(cz[r] >> 16));
    double part_g = fma(sc, acc, z * qsum);
#pragma unroll
    for (int m = 1; m < NG; m <<= 1) part_g += __shfl_xor(part_g, m, 64);
    if (i < n && g == 0) P.cand_scores[unit * n + i] = __double2ll_rn(part_g * 65536.0);
  }
}

__global__ __launch_bounds__(kUpdThreads) void vl_update_kernel(UpdParams P) {
  __shared__ unsigned long long key[kMaxCand];
  __shared__ int32_t pos[kMaxCand];         // candidate index -> position
  __shared__ uint8_t taken[kMaxCand];
  __shared__ uint8_t alive[kMaxCand];       // still tied with the threshold's digits so far
  __shared__ uint16_t freed[kMaxMoved];     // j-th freed VL slot
  __shared__ int32_t prom[kMaxMoved];       // j-th promoted position
  __shared__ int scan[kUpdThreads];
  __shared__ __align__(16) int hist[kBins];
  __shared__ int sel_digit, sel_need, sel_count;
  __shared__ unsigned long long red_mn[kUpdThreads / 64], red_mx[kUpdThreads / 64];
  __shared__ uint16_t list[64];             // the candidates still alive, once at most 64
  __shared__ int n_list, n_alive, key_bits;
  __shared__ unsigned long long key_min;
  __shared__ int n_freed_sh;
  const int64_t unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = P.k;
  const int n = k + static_cast<int>(P.nq - P.p0);
  int32_t *ui = P.idx + unit * k;

  // ---- candidates and their keys, and the range of the score keys
  int need = k;                             // still to take among the alive candidates
  {
    unsigned long long mn = ~0ull, mx = 0ull;
    for (int i = tid; i < n; i += kUpdThreads) {
      const int64_t p = i < k ? static_cast<int64_t>(ui[i]) : P.p0 + (i - k);
      const unsigned long long kv = order_key(P.scores[unit * P.stride + (P.by_cand ? i : p)]);
      pos[i] = static_cast<int32_t>(p);
      key[i] = kv;
      taken[i] = 0;
      alive[i] = 1;
      mn = kv < mn ? kv : mn;
      mx = kv > mx ? kv : mx;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const unsigned long long a = __shfl_xor(mn, m, 64), c = __shfl_xor(mx, m, 64);
      mn = a < mn ? a : mn;
      mx = c > mx ? c : mx;
    }
    if (lane == 0) {
      red_mn[tid >> 6] = mn;
      red_mx[tid >> 6] = mx;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kUpdThreads / 64; ++w) {
        mn = red_mn[w] < mn ? red_mn[w] : mn;
        mx = red_mx[w] > mx ? red_mx[w] : mx;
      }
      const unsigned long long x = mx - mn;
      key_min = mn;
      key_bits = 32 + (x ? 64 - __clzll(static_cast<long long>(x)) : 0);   // width of the rank keys
      n_alive = n;
      n_list = -1;                                                           // no pass has listed survivors
    }
    __syncthreads();
  }
  const unsigned long long kmin = key_min;

  // ---- radix select of the k best, most significant 12 bits first: each
  // pass counts the alive candidates per digit, finds the digit b* at which
  // the count from the top reaches `need`, takes the alive candidates above
  // it and keeps those equal to it alive (listing them). When the digit's
  // whole bucket is needed the selection is complete; when at most 64
  // candidates are left alive one wave ranks them directly.
  for (int top = key_bits; top > 0 && need > 0 && n_alive > 64;) {
    const int w = top < kDigitBits ? top : kDigitBits;
    const int sh = top - w;
    top = sh;
    for (int b = tid; b < kBins; b += kUpdThreads) hist[b] = 0;
    if (tid == 0) n_list = 0;
    __syncthreads();
    // one plain LDS atomic per alive candidate
    for (int i = tid; i < n; i += kUpdThreads)
      if (alive[i]) atomicAdd(&hist[rank_bits(key[i] - kmin, pos[i], sh, w)], 1);
    __syncthreads();
    if (tid < 64) {
      // lane l holds the 64 bins kBins - 1 - 64 l down to kBins - 64 (l + 1)
      constexpr int kPerLane = kBins / 64;
      const int hi_bin = kBins - 1 - kPerLane * lane;
      int tot = 0;
#pragma unroll
      for (int j = 0; j < kPerLane; j += 4) {
        const int4 c4 = *reinterpret_cast<const int4 *>(&hist[hi_bin - j - 3]);
        tot += c4.x + c4.y + c4.z + c4.w;
      }
      int incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      // the lane whose bins reach `need`, then its 64 bins one per lane
      const int cum = incl - tot;           // alive candidates in the bins above this lane's
      const unsigned long long hit = __ballot(cum < need && need <= incl);
      const int L = __ffsll(static_cast<long long>(hit)) - 1;           // exists: the bins hold >= need
      const int cum_l = __shfl(cum, L, 64);
      static_assert(kPerLane == 64, "one bin per lane in the second level");
      const int bin = kBins - 1 - kPerLane * L - lane;
      const int c = hist[bin];
      int ci = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(ci, off, 64);
        if (lane >= off) ci += v;
      }
      const int before = cum_l + ci - c;    // alive candidates in the bins above this one
      if (before < need && need <= before + c) {
        sel_digit = bin;
        sel_need = need - before;
        sel_count = c;
      }
    }
    __syncthreads();
    const uint32_t bstar = static_cast<uint32_t>(sel_digit);
    const bool whole = sel_need == sel_count;   // the bucket is needed entirely
    for (int i = tid; i < n; i += kUpdThreads) {
      if (!alive[i]) continue;
      const uint32_t dg = rank_bits(key[i] - kmin, pos[i], sh, w);
      if (dg > bstar || (dg == bstar && whole)) {
        taken[i] = 1;
        alive[i] = 0;
      } else if (dg < bstar) {
        alive[i] = 0;
      } else if (sel_count <= 64) {
        list[atomicAdd(&n_list, 1)] = static_cast<uint16_t>(i);
      }
    }
    need = whole ? 0 : sel_need;
    if (tid == 0) n_alive = whole ? 0 : sel_count;
    __syncthreads();
  }
  // at most 64 candidates left: lane l ranks the l-th of them by (score,
  // position) against the others; the best `need` are taken
  if (need > 0 && tid < 64) {
    // either the last pass listed its survivors, or no pass ran (n <= 64,
    // every candidate alive)
    const bool listed = n_list >= 0;
    const int cnt_alive = listed ? n_list : n;
    const int i = lane < cnt_alive ? (listed ? static_cast<int>(list[lane]) : lane) : 0;
    const unsigned long long ki = lane < cnt_alive ? key[i] : 0ull;
    const int32_t pi = lane < cnt_alive ? pos[i] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < cnt_alive; ++j) {
      const unsigned long long kj = __shfl(ki, j, 64);
      const int32_t pj = __shfl(pi, j, 64);
      rank += (kj > ki || (kj == ki && pj < pi)) ? 1 : 0;
    }
    if (lane < cnt_alive && rank < need) taken[i] = 1;
  }
  __syncthreads();

  // ---- flags: a freed slot (VL candidate not kept) or a promoted position
  // (recent candidate kept); one block scan ranks both in candidate order.
  // Exactly k candidates are kept, so the two counts are equal.
  constexpr int kPer = kMaxCand / kUpdThreads;
  const int c0 = tid * kPer;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = c0 + e;
    if (i < n) cnt += (i < k) ? !taken[i] : taken[i];
  }
  // block exclusive scan: inclusive within each wave, then the wave totals
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) scan[tid >> 6] = incl;
  __syncthreads();
  if (tid < 64) {
    const int wt = tid < kUpdThreads / 64 ? scan[tid] : 0;
    int wi = wt;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int v = __shfl_up(wi, off, 64);
      if (lane >= off) wi += v;
    }
    if (tid < kUpdThreads / 64) scan[64 + tid] = wi - wt;          // waves before this one
  }
  __syncthreads();
  const int excl = scan[64 + (tid >> 6)] + incl - cnt;
  // the freed count: the exclusive prefix at candidate k (k < n), found by
  // the thread whose run holds candidate k
  if (c0 <= k && k < c0 + kPer) {
    int f = excl;
    for (int i = c0; i < k; ++i) f += !taken[i];
    n_freed_sh = f;
  }
  __syncthreads();
  const int n_freed = n_freed_sh;
  const int64_t wbase = unit * P.words;
  int before = excl;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = c0 + e;
    if (i >= n) break;
    const int32_t p = pos[i];
    if (i < k && !taken[i]) {
      freed[before++] = static_cast<uint16_t>(i);
      atomicAnd(&P.bits[wbase + (p >> 5)], ~(1u << (p & 31)));      // back to its INT4 row
    } else if (i >= k && taken[i]) {
      prom[before - n_freed] = p;                                   // rank among the promoted
      ++before;
      atomicOr(&P.bits[wbase + (p >> 5)], 1u << (p & 31));          // promoted from the ring
    }
  }
  __syncthreads();
  for (int r = tid; r < n_freed; r += kUpdThreads) ui[freed[r]] = prom[r];

  // ---- the promoted rows, from the ring into the freed slots, 16 bytes per thread and step
  const int pieces = P.row_bytes / 16;
  for (int e = tid; e < n_freed * pieces; e += kUpdThreads) {
    const int r = e / pieces;
    const int c = e % pieces;
    const int slot = freed[r];
    const int64_t p = prom[r];
    // position T - W + j (j < 0) sits in ring row (win_offset + j) mod C
    const int64_t ring = (P.win_offset + (p - P.nq) + P.C) % P.C;
    const int64_t soff = (unit * P.C + ring) * P.row_bytes + 16 * c;
    const int64_t doff = (unit * k + slot) * P.row_bytes + 16 * c;
    *reinterpret_cast<uint4 *>(P.vl_k + doff) = *reinterpret_cast<const uint4 *>(P.ring_k + soff);
    *reinterpret_cast<uint4 *>(P.vl_v + doff) = *reinterpret_cast<const uint4 *>(P.ring_v + soff);
  }
}

}  // namespace
}  // namespace hq

using namespace hq;

namespace hq {
namespace {

// Checks shared by hq_vl_update and hq_vl_redetect; fills the common fields.
// Returns HQ_OK with *noop set when there is nothing to change.
hq_status prepare_update(const char *name, const hq_hybrid_kv *kv, int32_t *vl_idx, int64_t p0, UpdParams &P,
                         bool &noop) {
  noop = false;
  if (!kv) return fail(HQ_ERR_INVALID_ARG, "%s: null descriptor", name);
  if (kv->B < 1 || kv->Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "%s: B, Hkv must be >= 1", name);
  if (kv->D != 64 && kv->D != 128) return fail(HQ_ERR_UNSUPPORTED, "%s: D must be 64 or 128", name);
  if (!dtype_ok(kv->hp_dtype)) return fail(HQ_ERR_INVALID_ARG, "%s: bad dtype", name);
  if (kv->T < 1 || kv->W < 0 || kv->W > kv->T || kv->k < 0 || kv->k > kv->T - kv->W)
    return fail(HQ_ERR_INVALID_ARG, "%s: need 0 <= W <= T and 0 <= k <= T - W", name);
  const int64_t C = kv->win_cap > 0 ? kv->win_cap : kv->W;
  if (C < kv->W) return fail(HQ_ERR_INVALID_ARG, "%s: win_cap must be 0 or >= W", name);
  if (kv->W > 0 && (kv->win_offset < 0 || kv->win_offset >= C))
    return fail(HQ_ERR_INVALID_ARG, "%s: win_offset out of range", name);
  const int64_t nq = kv->T - kv->W;
  if (p0 > nq || p0 < 0 || p0 < kv->T - C)
    return fail(HQ_ERR_INVALID_ARG,
                "%s: p0 = %lld must lie in [max(0, T - win_cap), T - W] = [%lld, %lld]: only "
                "positions whose 16-bit rows are still in the ring can be promoted",
                name, static_cast<long long>(p0), static_cast<long long>(kv->T - C > 0 ? kv->T - C : 0),
                static_cast<long long>(nq));
  const int64_t n = kv->k + (nq - p0);
  if (nq - p0 > kMaxMoved)
    return fail(HQ_ERR_UNSUPPORTED, "%s: %lld positions left the window since p0, more than %d", name,
                static_cast<long long>(nq - p0), kMaxMoved);
  if (n > kMaxCand)
    return fail(HQ_ERR_UNSUPPORTED, "%s: %lld candidates per head exceed %d", name, static_cast<long long>(n),
                kMaxCand);
  if (kv->t_cap < nq || kv->t_cap % 32 != 0)
    return fail(HQ_ERR_INVALID_ARG, "%s: t_cap must be >= T - W and a multiple of 32", name);
  if (kv->k == 0 || nq == p0) { noop = true; return HQ_OK; }      // nothing to choose from or to change
  const int64_t units = static_cast<int64_t>(kv->B) * kv->Hkv;
  if (!vl_idx || !kv->vl_bits || !kv->vl_k || !kv->vl_v || !kv->win_k || !kv->win_v)
    return fail(HQ_ERR_INVALID_ARG, "%s: null pointer", name);
  const uintptr_t al = reinterpret_cast<uintptr_t>(kv->vl_k) | reinterpret_cast<uintptr_t>(kv->vl_v) |
                       reinterpret_cast<uintptr_t>(kv->win_k) | reinterpret_cast<uintptr_t>(kv->win_v);
  if (al % 16 || reinterpret_cast<uintptr_t>(kv->vl_bits) % 4 || reinterpret_cast<uintptr_t>(vl_idx) % 4)
    return fail(HQ_ERR_INVALID_ARG, "%s: misaligned buffer (rows 16 bytes, words and indices 4)", name);
  if (units > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "%s: too many heads", name);
  P = UpdParams{};
  P.idx = vl_idx;
  P.vl_k = static_cast<uint8_t *>(const_cast<void *>(kv->vl_k));
  P.vl_v = static_cast<uint8_t *>(const_cast<void *>(kv->vl_v));
  P.ring_k = static_cast<const uint8_t *>(kv->win_k);
  P.ring_v = static_cast<const uint8_t *>(kv->win_v);
  P.bits = const_cast<uint32_t *>(kv->vl_bits);
  P.words = kv->t_cap / 32;
  P.p0 = p0;
  P.nq = nq;
  P.k = kv->k;
  P.C = static_cast<int>(C);
  P.win_offset = kv->win_offset;
  P.row_bytes = kv->D * dtype_bytes(kv->hp_dtype);
  P.t_cap = kv->t_cap;
  P.Hkv = kv->Hkv;
  return HQ_OK;
}

}  // namespace
}  // namespace hq

extern "C" hq_status hq_vl_update(const hq_hybrid_kv *kv, int32_t *vl_idx, int64_t p0, const int64_t *scores,
                                  int64_t score_stride, void *stream) {
  UpdParams P;
  bool noop;
  hq_status s = prepare_update("hq_vl_update", kv, vl_idx, p0, P, noop);
  if (s != HQ_OK) return s;
  if (score_stride < kv->T - kv->W) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: score_stride < T - W");
  if (noop) { clear_error(); return HQ_OK; }
  if (!scores) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: null pointer");
  if (reinterpret_cast<uintptr_t>(scores) % 8) return fail(HQ_ERR_INVALID_ARG, "hq_vl_update: misaligned scores");
  P.scores = scores;
  P.stride = score_stride;
  const int64_t units = static_cast<int64_t>(kv->B) * kv->Hkv;
  hipLaunchKernelGGL(vl_update_kernel, dim3(static_cast<unsigned>(units)), dim3(kUpdThreads), 0, as_stream(stream),
                     P);
  return check_launch("hq_vl_update");
}

extern "C" size_t hq_vl_redetect_workspace_size(const hq_hybrid_kv *kv) {
  if (!kv || kv->B < 1 || kv->Hkv < 1 || kv->k < 0) return 0;
  return static_cast<size_t>(kv->B) * kv->Hkv * (static_cast<size_t>(kv->k) + kMaxMoved) * sizeof(int64_t);
}

extern "C" hq_status hq_vl_redetect(const hq_hybrid_kv *kv, int32_t *vl_idx, int64_t p0, const void *q_acc,
                                    hq_dtype q_dtype, int Hq, int R, void *ws, size_t ws_bytes, void *stream) {
  UpdParams P;
  bool noop;
  hq_status s = prepare_update("hq_vl_redetect", kv, vl_idx, p0, P, noop);
  if (s != HQ_OK) return s;
  if (!dtype_ok(q_dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: bad query dtype");
  if (q_dtype != kv->hp_dtype)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: the query dtype must be the cache's 16-bit dtype");
  if (Hq < 1 || Hq % kv->Hkv) return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: Hq must be a multiple of Hkv");
  if (R < 1 || R > 1024) return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: need 1 <= R <= 1024");
  if (noop) { clear_error(); return HQ_OK; }
  if (!q_acc || !kv->k_codes || !kv->k_sz) return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: null pointer");
  if (reinterpret_cast<uintptr_t>(q_acc) % 16 || reinterpret_cast<uintptr_t>(kv->k_codes) % 16 ||
      reinterpret_cast<uintptr_t>(kv->k_sz) % 4)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: misaligned buffer (ring and codes 16 bytes, scales 4)");
  const size_t need = hq_vl_redetect_workspace_size(kv);
  if (!ws || ws_bytes < need)
    return fail(HQ_ERR_WORKSPACE, "hq_vl_redetect: workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 8) return fail(HQ_ERR_INVALID_ARG, "hq_vl_redetect: misaligned workspace");
  const int64_t units = static_cast<int64_t>(kv->B) * kv->Hkv;
  const int64_t n = kv->k + (P.nq - p0);
  // candidates per round of a scoring block; rounds per block so that the
  // grid stays near 512 blocks (each block sums its head's query ring)
  const int64_t cpr = kUpdThreads / (kv->D / 32);
  const int64_t per_head = (n + cpr - 1) / cpr;
  int64_t rounds = (units * per_head + 511) / 512;
  rounds = rounds < 1 ? 1 : (rounds > kMaxRounds ? kMaxRounds : rounds);
  const int64_t blocks = units * ((n + cpr * rounds - 1) / (cpr * rounds));
  if (blocks > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_vl_redetect: too many heads");
  P.q_acc = q_acc;
  P.k_codes = static_cast<const uint8_t *>(kv->k_codes);
  P.k_sz = reinterpret_cast<const uint32_t *>(kv->k_sz);
  P.Hq = Hq;
  P.R = R;
  P.cand_scores = static_cast<int64_t *>(ws);
  hipStream_t st = as_stream(stream);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kUpdThreads);
  const int nr = static_cast<int>(rounds);
#define HQ_RD(DT_)                                                                                      \
  do {                                                                                                  \
    if (kv->D == 128) hipLaunchKernelGGL((redetect_scores_kernel<DT_, 128>), grid, block, 0, st, P, nr); \
    else hipLaunchKernelGGL((redetect_scores_kernel<DT_, 64>), grid, block, 0, st, P, nr);               \
  } while (0)
  if (q_dtype == HQ_F32) HQ_RD(HQ_F32);
  else if (q_dtype == HQ_BF16) HQ_RD(HQ_BF16);
  else HQ_RD(HQ_F16);
#undef HQ_RD
  s = check_launch("hq_vl_redetect (scores)");
  if (s != HQ_OK) return s;
  P.scores = P.cand_scores;
  P.stride = n;
  P.by_cand = 1;
  hipLaunchKernelGGL(vl_update_kernel, dim3(static_cast<unsigned>(units)), block, 0, st, P);
  return check_launch("hq_vl_redetect");
}
