// Hybrid-precision prefill attention (causal), on MFMA.
//
// What is computed: "HyQuant ... explained simply" (aifromscratch.in), The
// Technical Mechanics, Prefill Stage (the fused operator handles the
// quantized majority first, then overlays the 16-bit vertical-line tokens and
// the local window into the result); "Hybrid-precision attention reduces
// compute cost ..." (wpnews.pro), summary (queries are quantized as well as
// keys and values); kipquest.com paper page, The abstract (the prefill
// operator keeps vertical-line tokens and a local sliding window in full
// precision and quantizes the remaining context). For query position i of
// query head qh (KV head h = qh / G) and key position j <= i:
//   logit = q_i . k_j            if j is a VL position of h or i - W < j,
//   logit = q_hat_i . k_hat_j    otherwise,
// with q_hat, k_hat the INT4 round trip of the query and key rows in the KV
// cache format (per token, 32-channel groups, fp16 scale and zero); one causal
// softmax with scale sm_scale over all j <= i; P . V with the 16-bit V.
//
// Design (gfx950):
//  * A pre-pass encodes every query and key row exactly as the quantizer does
//    (hq_int4.h) and writes x_hat = s c + z (fp32) as two fp16 halves,
//    hi = fp16(x_hat) and lo = fp16(x_hat - hi). q_hat . k_hat is then
//    hi.hi + hi.lo + lo.hi on fp16 MFMA with fp32 accumulation, about 2^-21 from
//    the exact product (lo . lo is below that). One fp16 rounding of x_hat
//    (2^-11) would move the logits of the outlier channels far beyond the
//    output tolerance.
//  * The integer form (QF = 1, hq_prefill_attn_i8) runs the same product as
//    one int8 MFMA per 32-channel group over the codes plus one f16 MFMA for
//    the zero-point terms (codes_kernel below), and applies each group's
//    scale product per logit on the vector unit. It issues fewer than half
//    the matrix-core cycles but about twice the vector instructions; on
//    gfx950 the two forms take the same time.
//  * One workgroup = 4 waves = 128 query rows of one query head; wave w owns
//    rows 32w..32w+31. Per 32-key tile S^T = K . Q^T (v_mfma_f32_32x32x16):
//    lane l holds query l % 32 and 16 of the 32 keys, so the row softmax is
//    16 registers plus one exchange with lane l ^ 32. The exponentiated tile,
//    packed to fp16, is already the B operand of O^T += V^T . P^T: the
//    contraction index follows the accumulator's key order, and V^T is read
//    from LDS in that order (two 8-byte reads per fragment).
//  * Three key streams share one online softmax per row: the quantized keys
//    j <= i - W outside the VL set (split fp16 product), the window keys
//    i - W < j <= i and the VL keys j <= i - W gathered by index (16-bit
//    product). The three masks are disjoint and cover every j <= i once.
//  * K tiles are staged row-major in LDS; V tiles are staged transposed,
//    [d][key], in fp16 (bf16 inputs convert exactly for magnitudes in
//    [2^-17, 65504]; smaller ones round to the fp16 subnormal grid, absolute
//    error below 2^-25; larger ones are a precondition violation). The
//    probabilities are rounded to fp16 for the P . V MFMA (relative 2^-12).
//  * Query tiles are issued longest-first (the causal work grows with i).
#include <math.h>

#include <cmath>

#include "hq_common.h"
#include "hq_int4.h"

extern "C" hq_status hq_vl_bitmap(const int32_t *vl_idx, int n_heads, int k, int64_t t_cap,
                                  uint32_t *bits, void *stream);

namespace hq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Buffer view [base + off, base + bytes), empty when off >= bytes (off is
// wave-uniform and both are below 2^31: a signed max keeps it scalar); loads
// past the end of the view return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t view(const uint8_t *base, uint32_t bytes, uint32_t off) {
  const int32_t rem = static_cast<int32_t>(bytes) - static_cast<int32_t>(off);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base + off), static_cast<short>(0),
                                           rem > 0 ? rem : 0, 0x00020000);
}

constexpr int kD = 128;          // head_dim
constexpr int kBM = 128;         // query rows per workgroup
constexpr int kBN = 32;          // keys per tile
constexpr int kThreads = 256;
constexpr int kKPad = 8;         // halves of padding per K row in LDS
constexpr int kVPad = 4;         // halves of padding per V^T row in LDS
constexpr int kCPad = 16;        // bytes of padding per code row in LDS (integer form)
constexpr int kRPad = 8;         // halves of padding per zero-point operand row in LDS
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- pre-pass
// Four threads per (row, 32-channel group) of x [rows][D]; writes the split
// dequantized values of the same elements to hi and lo (fp16 bits).
template <int DT>
__global__ __launch_bounds__(256) void split_kernel(const void *__restrict__ x, uint32_t rows, int D,
                                                    uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
  const int ng = D / 32;
  const uint32_t total = rows * static_cast<uint32_t>(ng) * 4u;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;          // whole quads drop out together
  const int q = static_cast<int>(gid & 3u);
  const uint32_t item = gid >> 2;
  const int g = static_cast<int>(item % static_cast<uint32_t>(ng));
  const uint32_t r = item / static_cast<uint32_t>(ng);
  const int64_t src = static_cast<int64_t>(r) * D + g * 32 + q * 8;
  float v[8];
  load8<DT>(x, src, v);
  _Float16 s16, z16;
  const uint32_t packed = encode_quarter(v, s16, z16);
  const float s = static_cast<float>(s16), z = static_cast<float>(z16);
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float x0 = fmaf(s, static_cast<float>((packed >> (4 * e)) & 15u), z);
    const float x1 = fmaf(s, static_cast<float>((packed >> (4 * e + 4)) & 15u), z);
    const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
    const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
    const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
    wh[e / 2] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
    wl[e / 2] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
  }
  *reinterpret_cast<uint4 *>(hi + src) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  *reinterpret_cast<uint4 *>(lo + src) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
}

// Pre-pass of the integer form. Splitting every group of q_hat . k_hat,
//   sum_d (sq cq_d + zq)(sk ck_d + zk)
//     = sq sk C + zk (sq Cq + 32 zq) + zq (sk Ck),
// C = sum_d cq_d ck_d (an int8 MFMA over the codes), Cq and Ck the code sums,
// leaves per row and group: the scale, and the two rank-1 factors. Four
// threads per (row, group) of x [rows][128] write
//   codes [rows][128]  the codes as bytes,
//   sc                 keys [rows][4]: sk / 64; queries [rows][8]: sq 2^a for
//                      the four groups, then 2^(6 - a), the logit of one unit
//                      of the scaled score (fp32),
//   cor [rows][16]     the fp16 operands of one f16 MFMA that sums the
//                      zero-point terms of all four groups:
//                      queries [u_hi, u_lo, zq 2^a, zq 2^a], u = (sq Cq + 32 zq) 2^(a - 6),
//                      keys    [zk, zk, v_hi, v_lo],         v = sk Ck / 64,
// each a block of four (one per group), hi + lo the fp16 split of the fp32
// value. Products pair block by block: zk u_hi + zk u_lo + v_hi zq + v_lo zq,
// so the scores come out as 2^(a - 6) times the logits. The key side's 2^-6
// keeps v inside the fp16 range for inputs up to the fp16 maximum; the
// query row's power of two 2^a brings its largest operand just below 2^14,
// so small query groups stay clear of the fp16 subnormals (whose absolute
// error, times a key zero point near the fp16 maximum, would show in the
// logits).
template <int DT, bool QSIDE>
__global__ __launch_bounds__(256) void codes_kernel(const void *__restrict__ x, uint32_t rows,
                                                    uint8_t *__restrict__ codes, float *__restrict__ sc,
                                                    uint16_t *__restrict__ cor) {
  constexpr int ng = kD / 32;
  const uint32_t total = rows * static_cast<uint32_t>(ng) * 4u;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;          // whole quads drop out together
  const int q = static_cast<int>(gid & 3u);
  const uint32_t item = gid >> 2;
  const int g = static_cast<int>(item % static_cast<uint32_t>(ng));
  const uint32_t r = item / static_cast<uint32_t>(ng);
  const int64_t src = static_cast<int64_t>(r) * kD + g * 32 + q * 8;
  float v[8];
  load8<DT>(x, src, v);
  _Float16 s16, z16;
  const uint32_t packed = encode_quarter(v, s16, z16);
  uint32_t b0 = 0u, b1 = 0u;
  float csum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c0 = (packed >> (4 * e)) & 15u, c1 = (packed >> (16 + 4 * e)) & 15u;
    b0 |= c0 << (8 * e);
    b1 |= c1 << (8 * e);
    csum += static_cast<float>(c0 + c1);
  }
  *reinterpret_cast<uint2 *>(codes + src) = make_uint2(b0, b1);
  csum += quad_dpp<0xB1>(csum);                 // the group's code sum (exact)
  csum += quad_dpp<0x4E>(csum);
  const float s = static_cast<float>(s16);
  [[maybe_unused]] const float u = fmaf(s, csum, 32.f * static_cast<float>(z16));   // one rounding
  [[maybe_unused]] int a = 0;
  if constexpr (QSIDE) {
    // the row's four groups are 16 consecutive threads
    float m = fmaxf(fabsf(u) * 0x1p-6f, fabsf(static_cast<float>(z16)));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    if (m > 0.f) {
      int e;
      frexpf(m, &e);                         // m < 2^e
      a = 14 - e;
      a = a < -8 ? -8 : (a > 60 ? 60 : a);
    }
  }
  if (q != 0) return;
  const uint16_t zb = __builtin_bit_cast(uint16_t, z16);
  auto split = [](float w, uint16_t &hb, uint16_t &lb) {
    const _Float16 h = static_cast<_Float16>(w);
    hb = __builtin_bit_cast(uint16_t, h);
    lb = __builtin_bit_cast(uint16_t, static_cast<_Float16>(w - static_cast<float>(h)));
  };
  uint16_t *cr = cor + static_cast<int64_t>(r) * 16;
  uint16_t hb, lb;
  if constexpr (QSIDE) {
    float *sr = sc + static_cast<int64_t>(r) * 8;
    sr[g] = ldexpf(s, a);
    if (g == 0) *reinterpret_cast<float4 *>(sr + 4) = make_float4(ldexpf(1.f, 6 - a), 0.f, 0.f, 0.f);
    split(ldexpf(u, a - 6), hb, lb);
    const uint16_t za = __builtin_bit_cast(uint16_t, static_cast<_Float16>(ldexpf(static_cast<float>(z16), a)));
    cr[g] = hb;
    cr[4 + g] = lb;
    cr[8 + g] = za;
    cr[12 + g] = za;
  } else {
    sc[static_cast<int64_t>(r) * ng + g] = s * 0x1p-6f;
    split(s * csum * 0x1p-6f, hb, lb);          // exact in fp32
    cr[g] = zb;
    cr[4 + g] = zb;
    cr[8 + g] = hb;
    cr[12 + g] = lb;
  }
}

// 32-key tiles for the attention kernel, one thread per (tile, key, 8-channel
// chunk): row pos of src [heads][T][D] (16-bit) goes to V^T tile layout
// vt [heads][tiles][D][32] in fp16 and, when krows is given, to the row-major
// K tile layout krows [heads][tiles * 32][D] (16-bit). Key r of tile t is
// position 32 t + r, or idx[head][32 t + r] when idx is given (n_keys
// entries); keys past the end become zero rows.
template <int DT>
__global__ __launch_bounds__(256) void tile_kernel(const uint16_t *__restrict__ vsrc,
                                                   const uint16_t *__restrict__ ksrc, int64_t T,
                                                   const int32_t *__restrict__ idx, int n_keys, int tiles,
                                                   int heads, uint16_t *__restrict__ vt,
                                                   uint16_t *__restrict__ krows) {
  const int64_t total = static_cast<int64_t>(heads) * tiles * 32 * (kD / 8);
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % (kD / 8));
  const int64_t hr = gid / (kD / 8);             // (head, tile, key)
  const int r = static_cast<int>(hr % 32);
  const int64_t ht = hr / 32;                   // head * tiles + tile
  const int t = static_cast<int>(ht % tiles);
  const int64_t head = ht / tiles;
  const int key = t * 32 + r;
  int64_t pos = -1;
  if (idx) pos = key < n_keys ? idx[head * n_keys + key] : -1;
  else pos = key < T ? key : -1;
  uint4 u = make_uint4(0u, 0u, 0u, 0u), uk = u;
  if (pos >= 0) {
    u = *reinterpret_cast<const uint4 *>(vsrc + (head * T + pos) * kD + c * 8);
    if (krows) uk = *reinterpret_cast<const uint4 *>(ksrc + (head * T + pos) * kD + c * 8);
  }
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint16_t *dst = vt + (ht * kD + c * 8) * 32 + r;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    uint32_t f;
    if constexpr (DT == HQ_BF16) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      h2 v2 = {static_cast<_Float16>(bf16_to_f32(w[x] & 0xFFFFu)), static_cast<_Float16>(bf16_to_f32(w[x] >> 16))};
      f = __builtin_bit_cast(uint32_t, v2);
    } else {
      f = w[x];
    }
    dst[(2 * x) * 32] = static_cast<uint16_t>(f & 0xFFFFu);
    dst[(2 * x + 1) * 32] = static_cast<uint16_t>(f >> 16);
  }
  if (krows) *reinterpret_cast<uint4 *>(krows + (hr) * kD + c * 8) = uk;
}

// ---------------------------------------------------------------- attention
struct PrefillParams {
  const uint16_t *q;                // 16-bit [B][Hq][T][D]
  const uint16_t *k;                // 16-bit [B][Hkv][T][D]
  const uint16_t *q_hi, *q_lo;      // fp16 [B][Hq][T][D]
  const uint16_t *k_hi, *k_lo;      // fp16 [B][Hkv][T][D]
  const uint8_t *q_codes, *k_codes; // integer form (codes_kernel): codes [..][T][D]
  const float *q_sc, *k_sc;         //   group scales [..][T][4]
  const uint16_t *q_cor, *k_cor;    //   zero-point MFMA operands [..][T][16]
  const uint16_t *vt;               // fp16 V^T tiles [B][Hkv][ntk][D][32]
  const uint16_t *vl_k;             // 16-bit VL key rows [B][Hkv][nvt * 32][D]
  const uint16_t *vl_vt;            // fp16 VL V^T tiles [B][Hkv][nvt][D][32]
  const int32_t *vl_idx;            // [B][Hkv][k_vl], ascending
  const uint32_t *vl_bits;          // [B][Hkv][words]
  float *out;                       // [B][Hq][T][D]
  float *lse;                       // [B][Hq][T] or null
  int64_t T, words;
  int B, Hq, Hkv, G, W, k_vl, n_qt, ntk, nvt;
  float cs;                         // sm_scale * log2(e)
};

__device__ __forceinline__ f32x16 mfma_f16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                               c, 0, 0, 0);
}
template <int DT>
__device__ __forceinline__ f32x16 mfma_16bit(uint4 a, uint4 b, f32x16 c) {
  if constexpr (DT == HQ_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
  else
    return mfma_f16(a, b, c);
}
__device__ __forceinline__ i32x16 mfma_i8(u32x4 a, u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c,
                                               0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Stream kinds: quantized keys, window keys, VL keys.
enum { kQuant = 0, kWin = 1, kVl = 2 };

// The staged data of one 32-key tile: the keys (16-bit rows or the split
// planes, row-major and padded; or, in the integer form, the codes, group
// scales and zero-point operands) and the V^T tile ([d][key], padded).
// K tiles in two slots, V^T tiles and VL positions in three (see run_stream).
struct PrefillShared {
  union {
    struct {
      uint16_t ka[2][kBN][kD + kKPad];
      uint16_t kb[2][kBN][kD + kKPad];
    } f;
    struct {
      uint8_t kc[2][kBN][kD + kCPad];
      float ksc[2][kBN][4];
      uint16_t kcor[2][kBN][16 + kRPad];
    } i;
  } k;
  uint16_t vt[3][kD][kBN + kVPad];
  int32_t pos[3][kBN];
  int nvl;
};

// QF: the form of the quantized stream's q_hat . k_hat, 0 = three fp16
// passes over the split planes, 1 = int8 MFMA over the codes (integer form).
template <int DT, int QF>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams P) {
  __shared__ __align__(16) PrefillShared sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  // Block order: longest rows first. Workgroups go to the 8 XCDs round-robin
  // (block id mod 8); when the KV heads divide evenly, XCD x takes the KV
  // heads u = x, x + 8, ... with all their query heads, so every query head
  // and query tile in flight on an XCD that streams a KV head's tiles shares
  // them through that XCD's L2.
  int b, qh, qt;
  {
    const int U = P.B * P.Hkv;
    if (U % kNumXcd == 0) {
      const int x = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
      const int per = (U / kNumXcd) * P.G;              // (unit, query head) items per XCD and tile
      const int rem = j % per;
      const int unit = x + kNumXcd * (rem / P.G);
      b = unit / P.Hkv;
      qh = (unit % P.Hkv) * P.G + rem % P.G;
      qt = P.n_qt - 1 - j / per;
    } else {
      const int bq = blockIdx.x % (P.B * P.Hq);
      b = bq / P.Hq;
      qh = bq % P.Hq;
      qt = P.n_qt - 1 - blockIdx.x / (P.B * P.Hq);
    }
  }
  const int h = qh / P.G;
  const int64_t bh = static_cast<int64_t>(b) * P.Hkv + h;
  const int64_t q0 = static_cast<int64_t>(qt) * kBM;
  const int64_t qi = q0 + wave * 32 + (lane & 31);           // this lane's query position
  const bool q_ok = qi < P.T;
  const int64_t qrow = (static_cast<int64_t>(b) * P.Hq + qh) * P.T + (q_ok ? qi : P.T - 1);
  const int64_t qlast = (q0 + kBM - 1 < P.T - 1) ? q0 + kBM - 1 : P.T - 1;

  // running max of the raw logits; starts finite (the rescale runs before any
  // finite logit is used) and small enough that -cs * m_run stays finite
  float m_run = -1e30f;
  float l_run = 0.f;                 // this lane's share of the row sum
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  auto key_of = [&](int r) { return 8 * (r >> 2) + 4 * half + (r & 3); };

  // ---- one 32-key tile from LDS slot `sl`: mask, online softmax, P . V.
  // okm: this lane's valid keys of the tile as a bit mask over the register
  // key order c = 8 (r / 4) + (r % 4) (key 4 half + c); all_ok: the whole
  // tile is valid for every lane of the wave (no per-element mask); unit: the
  // logit of one unit of s (1, or the query row's 2^(6 - a) on the integer
  // form's stream; the same in both lanes of a query).
  auto consume = [&](f32x16 &s, int sl, uint32_t okm, bool all_ok, float unit) {
    if (!all_ok) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        s[r] = ((okm >> c) & 1u) ? s[r] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * unit;
    // the running max m_run is kept in raw logit units (before sm_scale, which
    // is positive); p = 2^(cs (unit s - m_run))
    if (__builtin_expect(__ballot(tmax > m_run) != 0, 0)) {
      const float mn = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(P.cs * (m_run - mn));
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float nm = -P.cs * m_run;
    const float cs = P.cs * unit;
    uint32_t pk[8];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], cs, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], cs, nm));
      ls += p0 + p1;
      pk[r / 2] = pack2_f16(p0, p1);
    }
    l_run += ls;
    const uint4 pf[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t *vrow = &sm.vt[sl][dt * 32 + (lane & 31)][0];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 a0 = *reinterpret_cast<const uint2 *>(vrow + 16 * c + 4 * half);
        const uint2 a1 = *reinterpret_cast<const uint2 *>(vrow + 16 * c + 8 + 4 * half);
        o[dt] = mfma_f16(make_uint4(a0.x, a0.y, a1.x, a1.y), pf[c], o[dt]);
      }
    }
  };
  // VL keys of a tile whose keys are all in range, from the tile's VL word
  // (wave-uniform): element r holds key c(r) in lanes 0-31 and key c(r) + 4 in
  // lanes 32-63, so each element's valid lanes form a 64-bit mask built on the
  // scalar unit and the select is a single v_cndmask per element.
  const float ninf = kNegInf;
  auto mask_vl_uniform = [&](f32x16 &s, uint32_t word) {
    const uint32_t nw = ~word;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 8 * (r >> 2) + (r & 3);
      const uint32_t lo = 0u - ((nw >> c) & 1u);
      const uint32_t hi = 0u - ((nw >> (c + 4)) & 1u);
      const uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
      asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(s[r]) : "v"(ninf), "s"(m));
    }
  };
  // bits c of the register key order for which key 4 half + c lies in (lo, hi]
  // (tile-relative keys; lo < hi)
  auto range_mask = [&](int lo, int hi) {
    lo -= 4 * half;
    hi -= 4 * half;
    const uint32_t upto = hi >= 31 ? 0xFFFFFFFFu : (hi < 0 ? 0u : ((2u << hi) - 1u));
    const uint32_t below = lo >= 31 ? 0xFFFFFFFFu : (lo < 0 ? 0u : ((2u << lo) - 1u));
    return upto & ~below;
  };
  // the first and last query rows of this wave
  const int64_t wq0 = q0 + wave * 32;
  const int64_t wq1 = (wq0 + 31 < P.T - 1) ? wq0 + 31 : P.T - 1;

  // ---- a stream of 32-key tiles t0 .. t1 - 1, staged through two LDS slots
  // with the next tile's global loads in flight during each tile's MFMAs
  struct Pre {
    u32x4 a[2], b[2], v[2];
    int32_t pos;
  };
  // scores of one tile as the MFMAs leave them: s (fp32), and in the integer
  // form the per-group int32 code products c (s then holds the zero-point sums)
  struct Acc {
    f32x16 s;
    i32x16 c[4];
  };
  // this lane's query in the integer form: codes of the four groups (its 16
  // bytes of each), zero-point operand (its 8 halves), group scales, the
  // logit of one unit of its scores
  struct QInt {
    u32x4 c[4];
    uint4 cor;
    float4 sc;
    float unit;
  } qn;
  auto run_stream = [&](const int kind, const int t0, const int t1, const uint4 (&fq0)[8],
                        const uint4 (&fq1)[8]) {
    if (t0 >= t1) return;
    const bool ints = QF == 1 && kind == kQuant;     // integer form
    const bool two = kind == kQuant && !ints;
    const uint16_t *kpa = kind == kQuant ? P.k_hi : (kind == kWin ? P.k : P.vl_k);
    const int64_t krows = kind == kVl ? static_cast<int64_t>(P.nvt) * kBN : P.T;   // rows per head
    const uint8_t *ka_base = reinterpret_cast<const uint8_t *>(kpa + bh * krows * kD);
    const uint8_t *kb_base = reinterpret_cast<const uint8_t *>(P.k_lo + bh * krows * kD);
    const uint32_t kbytes = static_cast<uint32_t>(krows) * kD * 2;
    const uint8_t *v_base = reinterpret_cast<const uint8_t *>(
        (kind == kVl ? P.vl_vt : P.vt) + bh * (kind == kVl ? P.nvt : P.ntk) * (kD * kBN));
    const uint32_t vbytes = static_cast<uint32_t>(kind == kVl ? P.nvt : P.ntk) * (kD * kBN) * 2;
    const int32_t *vl = P.vl_idx + bh * P.k_vl;
    // per-thread byte offsets inside a tile (K rows past the end read as 0)
    const uint32_t lk0 = threadIdx.x * 16, lk1 = (kThreads + threadIdx.x) * 16;
    auto load = [&](int t, Pre &L) {
      const uint32_t toff = static_cast<uint32_t>(t) * kBN * kD * 2;     // wave-uniform
      if (ints) {
        // a[0]: 16 bytes of codes; a[1]: a key's group scales (threads 0-31) or
        // half a zero-point operand row (threads 64-127)
        const uint32_t rows = static_cast<uint32_t>(P.T), t32 = static_cast<uint32_t>(t) * kBN;
        const __amdgpu_buffer_rsrc_t rc = view(P.k_codes + bh * P.T * kD, rows * kD, t32 * kD);
        L.a[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, lk0, 0, 0);
        if (threadIdx.x < kBN) {
          const __amdgpu_buffer_rsrc_t rs =
              view(reinterpret_cast<const uint8_t *>(P.k_sc + bh * P.T * 4), rows * 16, t32 * 16);
          L.a[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lk0, 0, 0);
        } else if (threadIdx.x >= 64 && threadIdx.x < 128) {
          const __amdgpu_buffer_rsrc_t rr =
              view(reinterpret_cast<const uint8_t *>(P.k_cor + bh * P.T * 16), rows * 32, t32 * 32);
          L.a[1] = __builtin_amdgcn_raw_buffer_load_b128(rr, (threadIdx.x - 64) * 16, 0, 0);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rka = view(ka_base, kbytes, toff);
        L.a[0] = __builtin_amdgcn_raw_buffer_load_b128(rka, lk0, 0, 0);
        L.a[1] = __builtin_amdgcn_raw_buffer_load_b128(rka, lk1, 0, 0);
        if (two) {
          const __amdgpu_buffer_rsrc_t rkb = view(kb_base, kbytes, toff);
          L.b[0] = __builtin_amdgcn_raw_buffer_load_b128(rkb, lk0, 0, 0);
          L.b[1] = __builtin_amdgcn_raw_buffer_load_b128(rkb, lk1, 0, 0);
        }
      }
      const __amdgpu_buffer_rsrc_t rv = view(v_base, vbytes, toff);
      L.v[0] = __builtin_amdgcn_raw_buffer_load_b128(rv, lk0, 0, 0);
      L.v[1] = __builtin_amdgcn_raw_buffer_load_b128(rv, lk1, 0, 0);
      L.pos = 0;
      if (kind == kVl && threadIdx.x < kBN) {
        const int j = t * kBN + static_cast<int>(threadIdx.x);
        L.pos = j < sm.nvl ? vl[j] : -1;
      }
    };
    auto store = [&](int ks, int vs, const Pre &L) {
      if (ints) {
        const int tx = threadIdx.x;
        *reinterpret_cast<u32x4 *>(&sm.k.i.kc[ks][tx >> 3][(tx & 7) * 16]) = L.a[0];
        if (tx < kBN) *reinterpret_cast<u32x4 *>(&sm.k.i.ksc[ks][tx][0]) = L.a[1];
        else if (tx >= 64 && tx < 128)
          *reinterpret_cast<u32x4 *>(&sm.k.i.kcor[ks][(tx - 64) >> 1][((tx - 64) & 1) * 8]) = L.a[1];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = e * kThreads + threadIdx.x;
        const int r = idx >> 4, c = idx & 15;
        if (!ints) *reinterpret_cast<u32x4 *>(&sm.k.f.ka[ks][r][c * 8]) = L.a[e];
        if (two) *reinterpret_cast<u32x4 *>(&sm.k.f.kb[ks][r][c * 8]) = L.b[e];
        const int d = idx >> 2, k8 = (idx & 3) * 8;       // V^T: row d, keys k8 .. k8 + 7
        *reinterpret_cast<u32x4 *>(&sm.vt[vs][d][k8]) = L.v[e];
      }
      if (kind == kVl && threadIdx.x < kBN) sm.pos[vs][threadIdx.x] = L.pos;
    };
    // the MFMAs of S^T for the tile in K slot ks
    auto qk = [&](int ks) {
      Acc acc;
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      if (ints) {
        // zero-point sums of all four groups (one f16 MFMA), then one int8
        // MFMA per 32-channel group over the codes
        const uint4 kr = *reinterpret_cast<const uint4 *>(&sm.k.i.kcor[ks][lane & 31][half * 8]);
        acc.s = mfma_f16(kr, qn.cor, sc);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          i32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0;
          const u32x4 kc = *reinterpret_cast<const u32x4 *>(&sm.k.i.kc[ks][lane & 31][g * 32 + half * 16]);
          acc.c[g] = mfma_i8(kc, qn.c[g], z);
        }
        return acc;
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const uint4 ah = *reinterpret_cast<const uint4 *>(&sm.k.f.ka[ks][lane & 31][kc * 16 + half * 8]);
        if (kind == kQuant) {
          const uint4 al = *reinterpret_cast<const uint4 *>(&sm.k.f.kb[ks][lane & 31][kc * 16 + half * 8]);
          sc = mfma_f16(ah, fq0[kc], sc);
          sc = mfma_f16(ah, fq1[kc], sc);
          sc = mfma_f16(al, fq0[kc], sc);
        } else {
          sc = mfma_16bit<DT>(ah, fq0[kc], sc);
        }
      }
      acc.s = sc;
      return acc;
    };
    // S^T of the tile in K slot ks from its MFMA results; in the integer form,
    // in the query row's units: s + sum_g (sq_g 2^a) (sk_g / 64) c_g, the
    // scales of this lane's query and of each register's key
    auto finish = [&](const Acc &acc, int ks) {
      if (!ints) return acc.s;
      f32x16 sc = acc.s;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float4 m = *reinterpret_cast<const float4 *>(&sm.k.i.ksc[ks][key_of(r)][0]);
        float x = sc[r];
        x = fmaf(static_cast<float>(acc.c[0][r]), qn.sc.x * m.x, x);
        x = fmaf(static_cast<float>(acc.c[1][r]), qn.sc.y * m.y, x);
        x = fmaf(static_cast<float>(acc.c[2][r]), qn.sc.z * m.z, x);
        x = fmaf(static_cast<float>(acc.c[3][r]), qn.sc.w * m.w, x);
        sc[r] = x;
      }
      return sc;
    };
    // Software pipeline, one barrier per tile: iteration i (tile t = t0 + i)
    // issues the score MFMAs of tile t + 1 (K slot (i + 1) % 2) before the
    // softmax and P . V of tile t (V slot i % 3), so the matrix core works
    // while the vector unit runs the softmax (the integer form's epilogue of
    // tile t + 1 follows the softmax of tile t), and stores tile t + 2 into K
    // slot i % 2 and V slot (i + 2) % 3, which no wave reads during iteration
    // i (their last readers finished before the previous barrier).
    Pre pa, pb;
    load(t0, pa);
    store(0, 0, pa);
    __syncthreads();
    if (t0 + 1 < t1) load(t0 + 1, pb);
    f32x16 s_cur = finish(qk(0), 0);
    if (t0 + 1 < t1) store(1, 1, pb);
    if (t0 + 2 < t1) load(t0 + 2, pa);
    __syncthreads();
    int vs = 0;                                  // V slot of tile t: i % 3
    // one tile; `st` holds tile t + 2 (loaded an iteration earlier), tile t + 3
    // goes into `ld`, so each tile's loads have a whole iteration to land
    auto iter = [&](const int t, const Pre &st, Pre &ld) {
      const int i = t - t0;
      const int vs2 = vs == 0 ? 2 : vs - 1;      // (i + 2) % 3
      if (t + 3 < t1) load(t + 3, ld);
      Acc a_next;
      if (t + 1 < t1) a_next = qk((i + 1) & 1);
      f32x16 &sv = s_cur;
      const int64_t k0 = static_cast<int64_t>(t) * kBN;
      if (kind == kQuant) {
        // keys k0 + m <= qi - W outside the VL set
        const uint32_t word = P.vl_bits[bh * P.words + t];         // VL bits of keys k0 .. k0 + 31
        // the VL keys: selects with scalar lane masks (all-ones when word == 0)
        mask_vl_uniform(sv, word);
        // the range j <= i - W: a per-lane mask only on tiles that cross it
        const bool in_range = k0 + kBN - 1 <= wq0 - P.W;           // wave-uniform
        uint32_t okm = 0u;
        if (!in_range) {
          const int hi = static_cast<int>(qi - P.W - k0 < 64 ? qi - P.W - k0 : 64);
          okm = range_mask(-1, hi);
        }
        consume(sv, vs, okm, in_range, ints ? qn.unit : 1.f);
      } else if (kind == kWin) {
        // keys qi - W < k0 + m <= qi
        const bool full = k0 > wq1 - P.W && k0 + kBN - 1 <= wq0;
        const int64_t lo64 = qi - P.W - k0, hi64 = qi - k0;
        const int lo = static_cast<int>(lo64 < -1 ? -1 : (lo64 > 64 ? 64 : lo64));
        const int hi = static_cast<int>(hi64 < -1 ? -1 : (hi64 > 64 ? 64 : hi64));
        consume(sv, vs, range_mask(lo, hi), full, 1.f);
      } else {
        uint32_t okm = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          const int64_t j = sm.pos[vs][4 * half + c];
          okm |= static_cast<uint32_t>(j >= 0 && j <= qi - P.W) << c;
        }
        consume(sv, vs, okm, false, 1.f);
      }
      f32x16 s_next;
      if (t + 1 < t1) s_next = finish(a_next, (i + 1) & 1);
      if (t + 2 < t1) store(i & 1, vs2, st);
      __syncthreads();
      s_cur = s_next;
      vs = vs == 2 ? 0 : vs + 1;
    };
    for (int t = t0; t < t1; t += 2) {
      iter(t, pa, pb);
      if (t + 1 < t1) iter(t + 1, pb, pa);
    }
  };

  // ---- stream 1: quantized keys j <= i - W outside the VL set
  {
    const int64_t nkeys = qlast - P.W + 1;                    // keys 0 .. qlast - W
    const int ntiles = nkeys > 0 ? static_cast<int>((nkeys + kBN - 1) / kBN) : 0;
    uint4 fqh[8], fql[8];
    if constexpr (QF == 0) {
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int64_t off = qrow * kD + kc * 16 + half * 8;
        fqh[kc] = *reinterpret_cast<const uint4 *>(P.q_hi + off);
        fql[kc] = *reinterpret_cast<const uint4 *>(P.q_lo + off);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        qn.c[g] = *reinterpret_cast<const u32x4 *>(P.q_codes + qrow * kD + g * 32 + half * 16);
      qn.cor = *reinterpret_cast<const uint4 *>(P.q_cor + qrow * 16 + half * 8);
      qn.sc = *reinterpret_cast<const float4 *>(P.q_sc + qrow * 8);
      qn.unit = P.q_sc[qrow * 8 + 4];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) fqh[kc] = fql[kc] = make_uint4(0u, 0u, 0u, 0u);   // not read
    }
    run_stream(kQuant, 0, ntiles, fqh, fql);
  }
  {
    uint4 fqr[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      fqr[kc] = *reinterpret_cast<const uint4 *>(P.q + qrow * kD + kc * 16 + half * 8);
    // ---- stream 2: window keys i - W < j <= i (16-bit)
    if (P.W > 0) {
      const int64_t jlo = (q0 - P.W + 1 > 0) ? q0 - P.W + 1 : 0;
      run_stream(kWin, static_cast<int>(jlo / kBN), static_cast<int>(qlast / kBN) + 1, fqr, fqr);
    }
    // ---- stream 3: VL keys j <= i - W (16-bit, gathered by index)
    if (P.k_vl > 0) {
      if (threadIdx.x == 0) {                 // VL positions <= qlast - W (ascending list)
        const int32_t *vl = P.vl_idx + bh * P.k_vl;
        int lo = 0, hi = P.k_vl;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (vl[mid] <= qlast - P.W) lo = mid + 1; else hi = mid;
        }
        sm.nvl = lo;
      }
      __syncthreads();
      const int nvl = sm.nvl;
      run_stream(kVl, 0, (nvl + kBN - 1) / kBN, fqr, fqr);
    }
  }

  // ---- output: lane holds query lane % 32, channels dt * 32 + key_of(r)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (q_ok) {
    const float inv = 1.f / l_tot;
    float *orow = P.out + qrow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int d = dt * 32 + key_of(r);
        *reinterpret_cast<float4 *>(orow + d) =
            make_float4(o[dt][r] * inv, o[dt][r + 1] * inv, o[dt][r + 2] * inv, o[dt][r + 3] * inv);
      }
    if (half == 0 && P.lse) P.lse[qrow] = (P.cs * m_run + log2f(l_tot)) * kLn2;
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PrefillWs {
  size_t q_hi, q_lo, k_hi, k_lo, vt, vl_k, vl_vt, bits, total;
  int ntk, nvt;
};
PrefillWs prefill_ws(int B, int Hq, int Hkv, int64_t T, int D, int k_vl) {
  PrefillWs L{};
  L.ntk = static_cast<int>((T + kBN - 1) / kBN);
  L.nvt = (k_vl + kBN - 1) / kBN;
  const size_t qn = static_cast<size_t>(B) * Hq * T * D * 2, kn = static_cast<size_t>(B) * Hkv * T * D * 2;
  const size_t vtn = static_cast<size_t>(B) * Hkv * L.ntk * kBN * D * 2;
  const size_t vln = static_cast<size_t>(B) * Hkv * L.nvt * kBN * D * 2;
  const size_t words = static_cast<size_t>((T + 31) / 32);
  L.q_hi = 0;
  L.q_lo = align_up(L.q_hi + qn, 256);
  L.k_hi = align_up(L.q_lo + qn, 256);
  L.k_lo = align_up(L.k_hi + kn, 256);
  L.vt = align_up(L.k_lo + kn, 256);
  L.vl_k = align_up(L.vt + vtn, 256);
  L.vl_vt = align_up(L.vl_k + vln, 256);
  L.bits = align_up(L.vl_vt + vln, 256);
  L.total = L.bits + static_cast<size_t>(B) * Hkv * words * 4;
  return L;
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" size_t hq_prefill_workspace_size(int B, int Hq, int Hkv, int64_t T, int D, int k_vl) {
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || D < 1 || k_vl < 0) return 0;
  return prefill_ws(B, Hq, Hkv, T, D, k_vl).total;
}

namespace hq {
namespace {

// Both forms of hq_prefill_attn; qf selects the quantized stream's product
// (0 split fp16, 1 integer form). The integer form keeps its codes, scales and
// zero-point operands inside the split planes' workspace regions.
hq_status prefill_run(const char *name, int qf, const void *q, const void *k, const void *v, hq_dtype dtype,
                      int B, int Hq, int Hkv, int64_t T, int D, int group, int W, const int32_t *vl_idx,
                      int k_vl, float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes,
                      void *stream) {
  if (dtype != HQ_BF16 && dtype != HQ_F16)
    return fail(HQ_ERR_UNSUPPORTED, "%s: dtype must be HQ_BF16 or HQ_F16", name);
  if (D != kD) return fail(HQ_ERR_UNSUPPORTED, "%s: D must be 128", name);
  if (group != 32) return fail(HQ_ERR_UNSUPPORTED, "%s: group must be 32", name);
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1) return fail(HQ_ERR_INVALID_ARG, "%s: sizes must be >= 1", name);
  if (Hq % Hkv) return fail(HQ_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0", name);
  if (W < 0 || k_vl < 0) return fail(HQ_ERR_INVALID_ARG, "%s: W and k must be >= 0", name);
  if (k_vl > T) return fail(HQ_ERR_INVALID_ARG, "%s: k exceeds T", name);
  if (!q || !k || !v || !out || (k_vl > 0 && !vl_idx)) return fail(HQ_ERR_INVALID_ARG, "%s: null pointer", name);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(out)) % 16)
    return fail(HQ_ERR_INVALID_ARG, "%s: q, k, v and out must be 16-byte aligned", name);
  // thread counts of the pre-pass stay below 2^31, and so do the byte sizes
  // of one head's planes (T * 256) that the attention kernel's buffer views take
  if (static_cast<double>(B) * Hq * T * (D / 32) * 4 > 2.0e9)
    return fail(HQ_ERR_UNSUPPORTED, "%s: too many query rows for one call", name);
  if (T >= (int64_t{1} << 23)) return fail(HQ_ERR_UNSUPPORTED, "%s: T must be below 2^23", name);
  const PrefillWs L = prefill_ws(B, Hq, Hkv, T, D, k_vl);
  if (!ws || ws_bytes < L.total)
    return fail(HQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", name, L.total, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HQ_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", name);
  hipStream_t st = as_stream(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint16_t *qh = reinterpret_cast<uint16_t *>(w8 + L.q_hi), *ql = reinterpret_cast<uint16_t *>(w8 + L.q_lo);
  uint16_t *kh = reinterpret_cast<uint16_t *>(w8 + L.k_hi), *kl = reinterpret_cast<uint16_t *>(w8 + L.k_lo);
  uint16_t *vt = reinterpret_cast<uint16_t *>(w8 + L.vt);
  uint16_t *vlk = reinterpret_cast<uint16_t *>(w8 + L.vl_k), *vlvt = reinterpret_cast<uint16_t *>(w8 + L.vl_vt);
  uint32_t *bits = reinterpret_cast<uint32_t *>(w8 + L.bits);
  const uint16_t *q16 = static_cast<const uint16_t *>(q), *k16 = static_cast<const uint16_t *>(k);
  const uint16_t *v16 = static_cast<const uint16_t *>(v);

  // integer form: codes in the hi region; scales, then zero-point operands,
  // in the lo region (32 + 32 bytes per query row, 16 + 32 per key row,
  // against the region's 256)
  const uint32_t qrows = static_cast<uint32_t>(static_cast<int64_t>(B) * Hq * T);
  const uint32_t krows = static_cast<uint32_t>(static_cast<int64_t>(B) * Hkv * T);
  uint8_t *qc = w8 + L.q_hi, *kc = w8 + L.k_hi;
  float *qsc = reinterpret_cast<float *>(w8 + L.q_lo), *ksc = reinterpret_cast<float *>(w8 + L.k_lo);
  uint16_t *qcor = reinterpret_cast<uint16_t *>(w8 + L.q_lo + static_cast<size_t>(qrows) * 32);
  uint16_t *kcor = reinterpret_cast<uint16_t *>(w8 + L.k_lo + static_cast<size_t>(krows) * 16);

  // pre-pass: Q and K in the form the quantized stream reads; V^T tiles; VL K
  // rows and V^T tiles
  const uint32_t qthreads = qrows * (D / 32) * 4, kthreads = krows * (D / 32) * 4;
  const int heads = B * Hkv;
  const int64_t vthreads = static_cast<int64_t>(heads) * L.ntk * kBN * (kD / 8);
  const int64_t lthreads = static_cast<int64_t>(heads) * L.nvt * kBN * (kD / 8);
#define HQ_PRE(DT_)                                                                                        \
  do {                                                                                                     \
    if (qf == 0) {                                                                                         \
      hipLaunchKernelGGL(split_kernel<DT_>, dim3((qthreads + 255) / 256), dim3(256), 0, st, q, qrows, D, qh, ql); \
      hipLaunchKernelGGL(split_kernel<DT_>, dim3((kthreads + 255) / 256), dim3(256), 0, st, k, krows, D, kh, kl); \
    } else {                                                                                               \
      hipLaunchKernelGGL((codes_kernel<DT_, true>), dim3((qthreads + 255) / 256), dim3(256), 0, st, q, qrows, qc, \
                         qsc, qcor);                                                                       \
      hipLaunchKernelGGL((codes_kernel<DT_, false>), dim3((kthreads + 255) / 256), dim3(256), 0, st, k, krows, kc, \
                         ksc, kcor);                                                                       \
    }                                                                                                      \
    hipLaunchKernelGGL(tile_kernel<DT_>, dim3(static_cast<unsigned>((vthreads + 255) / 256)), dim3(256), 0, st,   \
                       v16, nullptr, T, nullptr, 0, L.ntk, heads, vt, nullptr);                            \
    if (L.nvt > 0)                                                                                         \
      hipLaunchKernelGGL(tile_kernel<DT_>, dim3(static_cast<unsigned>((lthreads + 255) / 256)), dim3(256), 0, st, \
                         v16, k16, T, vl_idx, k_vl, L.nvt, heads, vlvt, vlk);                              \
  } while (0)
  if (dtype == HQ_BF16) HQ_PRE(HQ_BF16);
  else HQ_PRE(HQ_F16);
#undef HQ_PRE
  hq_status s = check_launch(name);
  if (s != HQ_OK) return s;
  // VL membership bitmap (no VL: an all-zero bitmap)
  s = hq_vl_bitmap(vl_idx, heads, k_vl, ((T + 31) / 32) * 32, bits, stream);
  if (s != HQ_OK) return s;

  PrefillParams P{};
  P.q = q16;
  P.k = k16;
  P.q_hi = qh; P.q_lo = ql; P.k_hi = kh; P.k_lo = kl;
  P.q_codes = qc; P.k_codes = kc; P.q_sc = qsc; P.k_sc = ksc; P.q_cor = qcor; P.k_cor = kcor;
  P.vt = vt; P.vl_k = vlk; P.vl_vt = vlvt;
  P.vl_idx = vl_idx;
  P.vl_bits = bits;
  P.out = out;
  P.lse = lse;
  P.T = T;
  P.words = (T + 31) / 32;
  P.B = B; P.Hq = Hq; P.Hkv = Hkv; P.G = Hq / Hkv; P.W = W; P.k_vl = k_vl;
  P.n_qt = static_cast<int>((T + kBM - 1) / kBM);
  P.ntk = L.ntk; P.nvt = L.nvt;
  P.cs = (sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(static_cast<float>(D))) * kLog2e;
  const unsigned blocks = static_cast<unsigned>(P.n_qt) * B * Hq;
  if (dtype == HQ_BF16) {
    if (qf == 0) hipLaunchKernelGGL((prefill_kernel<HQ_BF16, 0>), dim3(blocks), dim3(kThreads), 0, st, P);
    else hipLaunchKernelGGL((prefill_kernel<HQ_BF16, 1>), dim3(blocks), dim3(kThreads), 0, st, P);
  } else {
    if (qf == 0) hipLaunchKernelGGL((prefill_kernel<HQ_F16, 0>), dim3(blocks), dim3(kThreads), 0, st, P);
    else hipLaunchKernelGGL((prefill_kernel<HQ_F16, 1>), dim3(blocks), dim3(kThreads), 0, st, P);
  }
  return check_launch(name);
}

}  // namespace
}  // namespace hq

extern "C" hq_status hq_prefill_attn(const void *q, const void *k, const void *v, hq_dtype dtype, int B,
                                     int Hq, int Hkv, int64_t T, int D, int group, int W,
                                     const int32_t *vl_idx, int k_vl, float sm_scale, float *out,
                                     float *lse, void *ws, size_t ws_bytes, void *stream) {
  return prefill_run("hq_prefill_attn", 0, q, k, v, dtype, B, Hq, Hkv, T, D, group, W, vl_idx, k_vl, sm_scale,
                     out, lse, ws, ws_bytes, stream);
}

extern "C" hq_status hq_prefill_attn_i8(const void *q, const void *k, const void *v, hq_dtype dtype, int B,
                                        int Hq, int Hkv, int64_t T, int D, int group, int W,
                                        const int32_t *vl_idx, int k_vl, float sm_scale, float *out,
                                        float *lse, void *ws, size_t ws_bytes, void *stream) {
  return prefill_run("hq_prefill_attn_i8", 1, q, k, v, dtype, B, Hq, Hkv, T, D, group, W, vl_idx, k_vl,
                     sm_scale, out, lse, ws, ws_bytes, stream);
}
