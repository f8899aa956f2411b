// Decode-step attention over the hybrid KV cache, split over the context
// with a log-sum-exp merge, plus the VL membership bitmap builder.
//
// What is computed: "HyQuant ... Explained for Beginners" (aifromscratch.in),
// "How It Works" (three token sets: vertical lines and the last W tokens in
// 16 bits, the rest INT4) and "The Technical Mechanics", Decode Stage (the
// INT4 keys and values are dequantized inside the attention computation, on
// the fly, instead of in a separate pass); kipquest.com paper page, "The
// abstract" (decode fuses KV dequantization with attention). All three sets
// feed one softmax.
//
// Kernel design (gfx950, wave64). The points below describe the generic
// passes (any D, G, fp32 inputs), on the vector unit; for head_dim 128, a
// chunk of 4 query heads and 16-bit queries both passes run their products
// on the 4x4x4 matrix cores instead (int4_split_d128_g4, fp_rows_d128_g4).
//  * One workgroup = 4 waves = one (sequence b, KV head h, head chunk of HB
//    query heads, split) unit of work. A split is a contiguous range of INT4
//    positions or of 16-bit rows (VL rows, then window rows).
//  * INT4 keys, HQ_LAYOUT_ROWS: one 16-byte load = one 32-channel group of
//    one token; LPT = D/32 lanes per token, 64/LPT tokens per wave step, so a
//    wave reads one contiguous 1 KB block of codes per load.
//  * q . k without dequantizing k: a nibble pair is turned into a 16-bit
//    float pair (MAGIC + c0, MAGIC + c4) with one and-or (bf16 MAGIC = 128,
//    fp16 MAGIC = 1024, both exact), multiplied by the matching query pair with
//    v_dot2 (two products per lane op, fp32 accumulate), and
//    logit = s * (sum q c) + z * (sum q) with the MAGIC offset folded into
//    the accumulator's start value. Every unpacked key group is shared by the
//    HB query heads of the GQA group.
//  * softmax: per wave step, wave-wide max per head (lane shuffles), one
//    rescale of the running state when the max grows, p = 2^(l - m) with the
//    log2(e) and 1/sqrt(D) factors folded into the scale.
//  * P . V without dequantizing v: values use HQ_LAYOUT_TILE16, so lane
//    (channel pair j) loads 16 consecutive tokens of its two channels with
//    one 16-byte load; a token pair becomes the exact fp16 pair
//    (c_t - 8, c_t+1 - 8) (one and-or onto 1024 and one packed fp16
//    subtract) and is multiplied by the fp16 pair (p_t s_t, p_t+1 s_t+1) with
//    v_dot2. Centring the codes keeps the fp16 rounding of p s from adding a
//    bias proportional to the mean code; the zero point, as z + 8 s, is added
//    once per split from per-group sums of p (z + 8 s). No cross-lane
//    reduction over tokens is needed.
//  * Split partials (m, l, o) go to the workspace; a second small kernel
//    merges them per unit in split order: m* = max m_s,
//    L = sum 2^(m_s - m*) l_s, out = sum 2^(m_s - m*) o_s / L. (A
//    last-block merge inside the split kernel needs a device-scope release
//    per block, which on gfx950 writes back the XCD's L2 each time and costs
//    far more than one extra launch.)
//  * Blocks are numbered so that all splits of a KV head run on the same XCD
//    (dispatch is round-robin over the 8 XCDs), keeping the partials in one
//    L2 for the merge; when the head group has more than one chunk of query
//    heads (G = 8, 16), the chunks of each split are adjacent, so they run
//    together and each KV tile comes from HBM once, the other chunks' reads
//    hitting the L2. (Holding all 16 heads of a group in one workgroup, the
//    tile shared in registers, measured slower at the GLM-4-9B shape: each
//    16-token step becomes four times the vector work with too few waves to
//    cover it.)
#include <math.h>

#include <cmath>
#include <mutex>

#include "hq_common.h"
#include "hq_int4.h"

namespace hq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeParams {
  const void *q;
  const uint8_t *k_codes;
  const uint8_t *v_codes;
  const uint32_t *k_sz;     // {s, z} fp16 pairs as one word per (token, group)
  const uint32_t *v_sz;
  const uint32_t *vl_bits;
  const void *vl_k, *vl_v, *win_k, *win_v;
  float *out;
  float *lse;
  float2 *part_ml;          // [B][Hq][S]
  float *part_o;            // [B][Hq][S][D]
  int64_t t_cap;            // rows per head of the INT4 planes
  int64_t nq;               // T - W
  int64_t bits_words;       // words per head of vl_bits
  int k, W, win_offset;
  int win_cap;              // rows of the window ring (>= W)
  int B, Hkv, Hq, G, nhc;   // nhc = head chunks per KV head
  int S_q, S_vl, S_win, S;  // splits per unit: INT4, VL rows, window rows
  int64_t len_q;            // positions per INT4 split (multiple of 64)
  int len_vl, len_win;      // rows per 16-bit split (multiples of the wave step)
  int units;                // B * Hkv * nhc
  int blocks_used;          // units * S
  int blocks_per_xcd;
  int upx;                  // whole units per XCD when the grid splits evenly into them, else 0
  float cs;                 // sm_scale * log2(e)
  // per-step upkeep (hq_decode_step), run by extra blocks of the merge launch
  int merge_blocks;         // blocks of the merge itself
  int merge_per_xcd;        // ceil(merge_blocks / 8): the merge part of the grid is 8 times this
  int up_q;                 // blocks that copy q into the detector's query ring (0: none)
  uint8_t *q_ring;          // [B][Hq][R][D] of the query dtype
  int R, ring_slot;
  int evict;                // 1: pack the window's oldest row into INT4 row T - W
  uint8_t *ek_codes, *ev_codes;
  uint32_t *ek_sz, *ev_sz;
};

// ---------------------------------------------------------------- lane helpers
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// DPP lane moves (bound_ctrl: lanes without a source read 0)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowShl = 0x100;      // + n: lane i reads lane i + n of its row of 16
constexpr int kRowRor = 0x120;      // + n: rotate right by n within the row

// sum over the LPT lanes of a token (consecutive lanes), result in all of them
template <int LPT>
__device__ __forceinline__ float token_sum(float v) {
  v += dpp_f<kQuadXor1>(v);
  if constexpr (LPT == 4) v += dpp_f<kQuadXor2>(v);
  return v;
}
// max over the token slots of the wave (lanes with equal lane % LPT); every
// lane of a token holds the same value, so this is the max over all lanes
template <int LPT>
__device__ __forceinline__ float slots_max(float v) {
#pragma unroll
  for (int m = LPT; m < 16; m <<= 1) {
    if (m == 2) v = fmaxf(v, dpp_f<kRowRor + 2>(v));
    else if (m == 4) v = fmaxf(v, dpp_f<kRowRor + 4>(v));
    else v = fmaxf(v, dpp_f<kRowRor + 8>(v));
  }
  v = fmaxf(v, shfl_xor_f(v, 16));
  v = fmaxf(v, shfl_xor_f(v, 32));
  return v;
}
template <int FROM>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b),
                                         c, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}
template <int QT>
__device__ __forceinline__ float dot2_q(uint32_t a, uint32_t b, float c) {
  if constexpr (QT == HQ_BF16) return dot2_bf16(a, b, c);
  else return dot2_f16(a, b, c);
}

// two fp32 -> packed fp16, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
// packed fp16 add of two bit patterns (v_pk_add_f16)
__device__ __forceinline__ uint32_t centre_f16x2(uint32_t a, uint32_t b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) + __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ float lo_f16(uint32_t w) { return f16_to_f32(w & 0xFFFFu); }
__device__ __forceinline__ float hi_f16(uint32_t w) { return f16_to_f32(w >> 16); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// 32 channels of one query head starting at element `off`, as 16 raw pairs
template <int QT>
__device__ __forceinline__ void load_q32(const void *q, int64_t off, uint32_t (&w)[16]) {
  const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + off);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = p[i];
    w[4 * i + 0] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
  }
}
template <int QT>
__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  if constexpr (QT == HQ_BF16) return bf16_to_f32(h);
  else return f16_to_f32(h);
}

// Per-wave running softmax state for HB heads. acc_e/acc_o hold the channel
// pair (2*cp, 2*cp+1) of this lane (P . V accumulators, relative to m).
template <int HB>
struct WaveState {
  float m[HB];
  float l[HB];
  float acc_e[HB];
  float acc_o[HB];
};

constexpr int kMaxSplits = 256;
struct SharedMem {
  uint32_t ps[kWaves][4 * 4 * 16];      // [wave][h][g][pair]   (INT4 pass)
  float p[kWaves][4 * 32];              // [wave][h][slot]      (16-bit pass)
  float zo[kWaves][4][4];               // [wave][h][g] zero-point sums
  float bm[kWaves][4];
  float bl[kWaves][4];
  float bo[kWaves][4][128];
};

// Slow path of the online softmax: the wave max per head and the rescale of
// every running quantity, taken only when some new logit exceeds the running
// max (wave-uniform branch).
template <int HB, int LPT>
__device__ __forceinline__ void raise_max(const float (&lg)[HB], WaveState<HB> &st, float (&zl)[HB]) {
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const float mx = slots_max<LPT>(lg[hh]);
    const float mn = fmaxf(st.m[hh], mx);
    if (mn != st.m[hh]) {
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(st.m[hh] - mu);
      st.l[hh] *= alpha;
      st.acc_e[hh] *= alpha;
      st.acc_o[hh] *= alpha;
      zl[hh] *= alpha;
      st.m[hh] = mn;
    }
  }
}

// ---------------------------------------------------------------- INT4 pass
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave priority from the share of the split still to do (c of n chunks
// done, both wave-uniform). The instruction arbiter of a SIMD prefers the
// higher user priority and, among equals, the older wave; with equal
// priorities the first block on a CU runs ahead and the second finishes
// alone at low occupancy. Raising the priority of the wave that is further
// behind keeps co-resident waves abreast, so they finish together.
// Signed arithmetic (n < 2^28) keeps it on the scalar unit.
__device__ __forceinline__ void prio_by_remaining(uint32_t c, uint32_t n) {
  const int32_t ni = static_cast<int32_t>(n);
  const int32_t rem = ni - static_cast<int32_t>(c);
  if (rem * 2 > ni) __builtin_amdgcn_s_setprio(3);
  else if (rem * 4 > ni) __builtin_amdgcn_s_setprio(2);
  else if (rem * 8 > ni) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Buffer resource over [base, base + bytes): loads past the end return 0,
// so ragged tails need no branch, and offsets are 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
// The view [base + off, base + bytes), empty when off >= bytes. off is
// wave-uniform and both are below 2^31, so the size is a signed max with 0,
// which stays on the scalar unit (an unsigned saturating subtract would be a
// vector instruction and put the descriptor in vector registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t view(const uint8_t *base, uint32_t bytes, uint32_t off) {
  const int32_t rem = static_cast<int32_t>(bytes) - static_cast<int32_t>(off);
  return make_rsrc(base + off, static_cast<uint32_t>(rem > 0 ? rem : 0));
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// non-temporal: the codes are streamed once per step
__device__ __forceinline__ u32x4 bload16nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// (x & m) | o in one instruction; m is wave-uniform (SGPR), o in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

// The 16 tokens of one channel pair of a TILE16 value tile (4 words; word a
// holds tokens 4a, 4a+2, 4a+1, 4a+3 in bytes 0..3) as centred fp16 pairs:
// e[i] = (c - 8) of channel 2cp for tokens (2i, 2i+1), o[i] = 16 (c - 8) of
// channel 2cp+1. A nibble ORed under the fp16 exponent of 1024 gives 1024 + c
// (low nibble) or 1024 + 16 c (high nibble), and one packed subtract of 1032
// or 1152 centres it exactly.
__device__ __forceinline__ void unpack_v_tile(const uint32_t (&vw)[4], uint32_t vmagic, uint32_t (&e)[8],
                                              uint32_t (&o)[8]) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t w0 = vw[a], w8 = vw[a] >> 8;
    e[2 * a] = centre_f16x2(and_or(w0, 0x000F000Fu, vmagic), 0xE408E408u);
    o[2 * a] = centre_f16x2(and_or(w0, 0x00F000F0u, vmagic), 0xE480E480u);
    e[2 * a + 1] = centre_f16x2(and_or(w8, 0x000F000Fu, vmagic), 0xE408E408u);
    o[2 * a + 1] = centre_f16x2(and_or(w8, 0x00F000F0u, vmagic), 0xE480E480u);
  }
}

template <int D>
struct Int4Loads {
  u32x4 kc;                 // 32 key codes of this lane's (token, group)
  uint32_t ks, vs;          // {s, z} of the key / value group
  uint32_t bits;            // VL bitmap word of this token
  u32x4 vc;                 // 16 tokens of this lane's value channel pair
};

template <int D, int HB, int QT>
__device__ void int4_split(const DecodeParams &P, SharedMem &sm, int b, int h, int i0,
                           int64_t r0, int64_t r1, WaveState<HB> &st) {
  constexpr int LPT = D / 32;          // lanes per token (one group each)
  constexpr int SLOTS = 64 / LPT;      // tokens per wave step
  constexpr int CP = D / 2;            // channel pairs
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int slot = lane / LPT;
  const int g = lane % LPT;
  const int cp = lane % CP;
  const int sub = lane / CP;           // 16-token sub-tile for the P.V lanes
  const int gp = cp / 16;
  const int64_t head = static_cast<int64_t>(b) * P.Hkv + h;

  // query pairs of this lane's group: qp[hh][j][m] = (q[8j+m], q[8j+m+4])
  uint32_t qp[HB][4][4];
  float qf[HB][32];
  float qsum[HB], negmq[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const int64_t qoff = (static_cast<int64_t>(b) * P.Hq + i0 + hh) * D + g * 32;
    float v[32];
    if constexpr (QT == HQ_F32) {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(P.q) + qoff);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = p[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
      uint32_t raw[16];
      load_q32<QT>(P.q, qoff, raw);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        v[2 * c] = half_bits_to_f32<QT>(raw[c] & 0xFFFFu);
        v[2 * c + 1] = half_bits_to_f32<QT>(raw[c] >> 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int a = 8 * j + m, c = 8 * j + m + 4;
          const uint32_t lo = (raw[a >> 1] >> (16 * (a & 1))) & 0xFFFFu;
          const uint32_t hi = (raw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
          qp[hh][j][m] = lo | (hi << 16);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) s += v[c];
    qsum[hh] = s;
    if constexpr (QT == HQ_F32) {
#pragma unroll
      for (int c = 0; c < 32; ++c) qf[hh][c] = v[c];
    }
  }
  constexpr uint32_t kMagic = (QT == HQ_BF16) ? 0x43004300u : 0x64006400u;
  constexpr float kMagicVal = (QT == HQ_BF16) ? 128.f : 1024.f;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) negmq[hh] = -kMagicVal * qsum[hh];
  const uint32_t magic = kMagic;           // held in a VGPR for v_and_or_b32
  const uint32_t vmagic = 0x64006400u;

  float zl[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) zl[hh] = 0.f;

  // buffer views of this split (loads past r1 return 0)
  const uint32_t n = static_cast<uint32_t>(r1 - r0);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(P.k_codes + (head * P.t_cap + r0) * (D / 2), n * (D / 2));
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(P.k_sz + (head * P.t_cap + r0) * (D / 32), n * (D / 8));
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(P.v_sz + (head * P.t_cap + r0) * (D / 32), n * (D / 8));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(P.v_codes + (head * P.t_cap + r0) * (D / 2),
                                              ((n + 15) / 16) * (CP * 16));
  const uint32_t w_first = static_cast<uint32_t>(r0 >> 5);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(P.vl_bits + head * P.bits_words + w_first,
                                              static_cast<uint32_t>(((r1 + 31) >> 5) - w_first) * 4);
  const uint32_t r0_bit = static_cast<uint32_t>(r0 & 31);

  auto issue = [&](uint32_t c, Int4Loads<D> &L) {
    const uint32_t tok = static_cast<uint32_t>(c) * SLOTS + slot;      // local token
    L.kc = bload16(rk, tok * (D / 2) + g * 16);
    L.ks = bload4(rks, tok * (D / 8) + g * 4);
    L.vs = bload4(rvs, tok * (D / 8) + g * 4);
    L.bits = bload4(rb, ((r0_bit + tok) >> 5) * 4);
    const uint32_t vt = static_cast<uint32_t>(c) * (SLOTS / 16) + sub;  // local tile
    L.vc = bload16(rv, vt * (CP * 16) + cp * 16);
  };

  // NPF-deep prefetch ring: while a wave works on one step, the loads of the
  // next NPF - 1 steps of that wave are in flight (the ring is unrolled so
  // every buffer stays in fixed registers).
  constexpr int NPF = 3;
  const uint32_t nsteps = (n + SLOTS - 1) / SLOTS;
  Int4Loads<D> ring[NPF];
#pragma unroll
  for (int jr = 0; jr < NPF; ++jr) {
    issue(wave + jr * kWaves, ring[jr]);
    __builtin_amdgcn_sched_barrier(0);   // keep the ring's issue order: waits are counts
  }
  // one wave step over chunk c held in `cur`
  auto step = [&](const uint32_t c, const Int4Loads<D> &cur) {
    const uint32_t tok = static_cast<uint32_t>(c) * SLOTS + slot;

    // ---- q . k (k never dequantized: s * sum(q c) + z * sum(q))
    float part[HB];
    const uint32_t w[4] = {cur.kc.x, cur.kc.y, cur.kc.z, cur.kc.w};
    if constexpr (QT == HQ_F32) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) part[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cv = static_cast<float>((w[j] >> (4 * e)) & 15u);
#pragma unroll
          for (int hh = 0; hh < HB; ++hh) part[hh] = fmaf(qf[hh][8 * j + e], cv, part[hh]);
        }
    } else {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) part[hh] = negmq[hh];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x0 = and_or(w[j], 0x000F000Fu, magic);
        const uint32_t x1 = and_or(w[j] >> 4, 0x000F000Fu, magic);
        const uint32_t x2 = and_or(w[j] >> 8, 0x000F000Fu, magic);
        const uint32_t x3 = and_or(w[j] >> 12, 0x000F000Fu, magic);
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          part[hh] = dot2_q<QT>(qp[hh][j][0], x0, part[hh]);
          part[hh] = dot2_q<QT>(qp[hh][j][1], x1, part[hh]);
          part[hh] = dot2_q<QT>(qp[hh][j][2], x2, part[hh]);
          part[hh] = dot2_q<QT>(qp[hh][j][3], x3, part[hh]);
        }
      }
    }
    const float ssc = lo_f16(cur.ks) * P.cs;
    const float zsc = hi_f16(cur.ks) * P.cs;
    const bool live = (tok < n) && !((cur.bits >> ((r0_bit + tok) & 31)) & 1u);
    float lg[HB];
    bool exceed = false;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float v = token_sum<LPT>(fmaf(ssc, part[hh], zsc * qsum[hh]));
      lg[hh] = live ? v : kNegInf;
      exceed |= lg[hh] > st.m[hh];
    }
    if (__ballot(exceed)) raise_max<HB, LPT>(lg, st, zl);

    // V scale and the zero point of the centred codes, z + 8 s; zero for
    // masked tokens (their planes may hold anything, NaN included)
    const float sv = live ? lo_f16(cur.vs) : 0.f;
    const float zv = live ? fmaf(8.f, lo_f16(cur.vs), hi_f16(cur.vs)) : 0.f;
    _Float16 *psh = reinterpret_cast<_Float16 *>(&sm.ps[wave][0]);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float mu = (st.m[hh] == kNegInf) ? 0.f : st.m[hh];
      const float p = fast_exp2(lg[hh] - mu);
      st.l[hh] += p;
      zl[hh] = fmaf(p, zv, zl[hh]);
      psh[(hh * LPT + g) * 32 + slot] = static_cast<_Float16>(p * sv);
    }
    wave_sync();

    // ---- p . v (v never dequantized: sum (p s)(c - 8), zero point later)
    const uint32_t vw[4] = {cur.vc.x, cur.vc.y, cur.vc.z, cur.vc.w};
    uint32_t e[8], o[8];
    unpack_v_tile(vw, vmagic, e, o);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const uint4 *src = reinterpret_cast<const uint4 *>(&sm.ps[wave][(hh * LPT + gp) * 16 + 8 * sub]);
      const uint4 pa = src[0], pb = src[1];
      const uint32_t pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        st.acc_e[hh] = dot2_f16(pr[i], e[i], st.acc_e[hh]);
        st.acc_o[hh] = dot2_f16(pr[i], o[i], st.acc_o[hh]);
      }
    }
  };
  // full groups of NPF steps: every refill is issued unconditionally (past
  // the split the buffer loads return 0), so each wait for the oldest ring
  // entry is a fixed count on every path into the loop
  uint32_t cb = wave;
  for (; cb + (NPF - 1) * kWaves < nsteps; cb += NPF * kWaves) {
#pragma unroll
    for (int jr = 0; jr < NPF; ++jr) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
      issue(cb + jr * kWaves + NPF * kWaves, ring[jr]);
    }
  }
  // the last NPF - 1 steps at most
#pragma unroll
  for (int jr = 0; jr < NPF - 1; ++jr)
    if (cb + jr * kWaves < nsteps) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
    }

  // ---- per-(head, group) zero-point sums, folded into the accumulators
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const float z = xor_sum<LPT>(zl[hh]);
    if (slot == 0) sm.zo[wave][hh][g] = z;
  }
  wave_sync();
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    float ae = st.acc_e[hh], ao = st.acc_o[hh];
    if constexpr (CP < 64) {       // D = 64: two 16-token sub-tiles share the channels
      ae += shfl_xor_f(ae, 32);
      ao += shfl_xor_f(ao, 32);
    }
    const float z = sm.zo[wave][hh][gp];
    st.acc_e[hh] = ae + z;
    st.acc_o[hh] = ao * 0.0625f + z;
    st.l[hh] = xor_sum<1>(st.l[hh]) * (1.0f / LPT);
  }
}

// ---------------------------------------------------------------- INT4 pass, D = 128, 4 heads
// Specialisation of the INT4 pass for the common shape (head_dim 128, a GQA
// chunk of 4 query heads, 16-bit queries). Both products run on the matrix
// cores with v_mfma_f32_4x4x4_16b_f16: sixteen independent 4x4 blocks per
// instruction, each lane feeding one row of A and one column of B of its
// block (lane 4 blk + i) and receiving that column of D in four registers
// (rows 0..3).
//
// Q . K: block blk = 4 g + tq computes, for key group g and the four tokens
// 4 tq .. 4 tq + 3 of the chunk, the four heads' group dots: A rows are the
// heads' query channels of group g, B columns the tokens' key codes. Lane
// (token t = lane % 16, group g = lane / 16) loads its own 32 codes, so every
// lane's D holds the four heads of its (token, group). Eight instructions
// cover the 32 channels of a group. Key codes become fp16 pairs without
// shifts at two nibble positions: the low nibble of each byte under the
// magic 1024 (ulp 1, so 1024 + c) and the high nibble in place under the
// magic 64 (ulp 1/16 at bits 4-7, so 64 + c); one shift by 8 serves the
// other two nibbles. The queries are rounded to fp16 once (exact for bf16
// magnitudes in [2^-17, 65504]; the fast path requires |q| < 65504) and the
// accumulation starts from minus the offsets, -(1024 sum of the low-nibble
// channels + 64 sum of the others), so it ends at q . c. The group scale and
// zero point are applied per (token, group) on the vector unit, and three
// permlane swaps with three adds sum the four groups (rows of 16 lanes) so
// that lane (t, h = lane / 16) holds the logit of head h for token t.
//
// P . V: block blk computes, for 4 value channels of one group, the four
// heads' sums over 4 tokens: A rows are the heads' weights p s of the
// tokens (written to LDS by the softmax lanes, 2 reads per lane), B columns
// the channels' centred codes from the TILE16 tiles. Lane l's D is then the
// four heads of channel 2l (even set) or 2l + 1 (odd set): the accumulator
// layout of the 16-bit pass.
typedef _Float16 h4x __attribute__((ext_vector_type(4)));
typedef float f4x __attribute__((ext_vector_type(4)));
typedef uint32_t u2x __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f4x mfma4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f4x c) {
  const u2x a = {a0, a1}, bb = {b0, b1};
  return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4x, a), __builtin_bit_cast(h4x, bb), c, 0, 0, 0);
}
// In-place row swaps between two registers (rows of 16 lanes): 32-swap
// exchanges rows 2,3 of x with rows 0,1 of y, 16-swap the odd rows of x with
// the even rows of y. Written as inline asm with both operands tied: the
// compiler's builtins for these instructions fold swap(x, x) to (x, x) and
// take both results from one register. The compiler does not see inside the
// asm, so it carries its own wait states: two before (a vector write of
// either operand just before) and two after (a read of the results).
__device__ __forceinline__ void permlane32_swap(float &x, float &y) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void permlane16_swap(float &x, float &y) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
// x of rows 0 + 2 and 1 + 3 in rows 0, 1; y of rows 0 + 2 and 1 + 3 in rows 2, 3
__device__ __forceinline__ float swap32_sum(float x, float y) {
  permlane32_swap(x, y);
  return x + y;
}
// x of rows 0 + 1 in row 0, y of rows 0 + 1 in row 1, x of rows 2 + 3 in row 2, y in row 3
__device__ __forceinline__ float swap16_sum(float x, float y) {
  permlane16_swap(x, y);
  return x + y;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kRowRor + 8>(v));
  v = fmaxf(v, dpp_f<kRowRor + 4>(v));
  v = fmaxf(v, dpp_f<kRowRor + 2>(v));
  return fmaxf(v, dpp_f<kRowRor + 1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kRowRor + 8>(v);
  v += dpp_f<kRowRor + 4>(v);
  v += dpp_f<kRowRor + 2>(v);
  return v + dpp_f<kRowRor + 1>(v);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
constexpr int kQuadBcast[4] = {0x00, 0x55, 0xAA, 0xFF};        // quad_perm [h,h,h,h]

template <int QT>
__device__ void int4_split_d128_g4(const DecodeParams &P, SharedMem &sm, int b, int h, int i0,
                                   int64_t r0, int64_t r1, WaveState<4> &st) {
  constexpr int D = 128, SLOTS = 16, CP = 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int t = lane & 15;             // token of the chunk
  const int row = lane >> 4;           // key group (loads, Q . K), head (softmax)
  const int hq = lane & 3;             // head of this lane's A row in Q . K and P . V
  const int64_t head = static_cast<int64_t>(b) * P.Hkv + h;

  // raw query channels of head hq, group `row`, loaded before the ring so
  // that their wait does not cover the ring's loads
  uint32_t qraw[16];
  load_q32<QT>(P.q, (static_cast<int64_t>(b) * P.Hq + i0 + hq) * D + row * 32, qraw);
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t vmagic = 0x64006400u;
  float zl[4] = {0.f, 0.f, 0.f, 0.f};   // sum p_h (z + 8 s) of group `row`, head h
  float lown = 0.f;                      // sum of p of head `row`
  // running max of head `row`; starts finite, so p = 2^(l - m) needs no
  // guard (a live logit above it always takes the rescale first)
  float mown = -__FLT_MAX__;

  // Each chunk gets its own buffer views, built in SGPRs from wave-uniform
  // offsets: the per-lane offsets below never change, so the loads need no
  // vector address arithmetic, and a view past the end of the split is empty
  // (its loads return 0). Splits start at multiples of 64 positions, so the
  // VL bits of chunk c sit in word c / 2 at bit 16 (c % 2) + t, and c % 2
  // equals wave % 2 for every chunk of this wave.
  const uint32_t n = static_cast<uint32_t>(r1 - r0);
  const int64_t row0 = head * P.t_cap + r0;
  const uint8_t *kb = P.k_codes + row0 * (D / 2);
  const uint8_t *ksb = reinterpret_cast<const uint8_t *>(P.k_sz + row0 * (D / 32));
  const uint8_t *vsb = reinterpret_cast<const uint8_t *>(P.v_sz + row0 * (D / 32));
  const uint8_t *vb = P.v_codes + row0 * (D / 2);
  const uint8_t *bb = reinterpret_cast<const uint8_t *>(P.vl_bits + head * P.bits_words + (r0 >> 5));
  const uint32_t nk = n * (D / 2), ns = n * (D / 8), nv = ((n + 15) / 16) * (CP * 16);
  const uint32_t nb = ((n + 31) >> 5) * 4;
  const uint32_t lo_k = t * (D / 2) + row * 16;
  const uint32_t lo_s = t * (D / 8) + row * 4;
  const uint32_t lo_v = lane * 16;
  const uint32_t bitpos = (wave & 1) * 16 + t;

  auto issue = [&](uint32_t c, Int4Loads<D> &L) {
    const uint32_t os = c * (SLOTS * D / 8);
    L.kc = bload16nt(view(kb, nk, c * (SLOTS * D / 2)), lo_k);
    L.ks = bload4(view(ksb, ns, os), lo_s);
    L.vs = bload4(view(vsb, ns, os), lo_s);
    L.bits = bload4(view(bb, nb, (c >> 1) * 4), 0);
    L.vc = bload16nt(view(vb, nv, c * (CP * 16)), lo_v);
  };

  // a 2-deep ring: one chunk's loads in flight while the wave works on the
  // other (deeper rings measured slower at every shape)
  constexpr int NPF = 2;
  const uint32_t nsteps = (n + SLOTS - 1) / SLOTS;
  Int4Loads<D> ring[NPF];
#pragma unroll
  for (int jr = 0; jr < NPF; ++jr) {
    issue(wave + jr * kWaves, ring[jr]);
    __builtin_amdgcn_sched_barrier(0);   // keep the ring's issue order: waits are counts
  }
  // fp16 query pairs in the order of the unpacked code pairs, while the
  // ring's first loads fly: qa[w][m] = channels (8w + m, 8w + m + 4)
  uint32_t qa[4][4];
  float nf, cq;
  {
    uint32_t hb[32];
    float se = 0.f, so = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const uint32_t bits = (qraw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
      _Float16 q16;
      if constexpr (QT == HQ_BF16) q16 = static_cast<_Float16>(bf16_to_f32(bits));
      else q16 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits));
      hb[c] = __builtin_bit_cast(uint16_t, q16);
      if (c & 1) so += static_cast<float>(q16);
      else se += static_cast<float>(q16);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int m = 0; m < 4; ++m) qa[w][m] = hb[8 * w + m] | (hb[8 * w + m + 4] << 16);
    cq = P.cs * (se + so);
    nf = -fmaf(1024.f, se, 64.f * so);
  }
  // per head i of this lane's group (the quad's lane i holds head i)
  f4x nofv;
  float cqv[4];
  nofv[0] = dpp_f<kQuadBcast[0]>(nf); cqv[0] = dpp_f<kQuadBcast[0]>(cq);
  nofv[1] = dpp_f<kQuadBcast[1]>(nf); cqv[1] = dpp_f<kQuadBcast[1]>(cq);
  nofv[2] = dpp_f<kQuadBcast[2]>(nf); cqv[2] = dpp_f<kQuadBcast[2]>(cq);
  nofv[3] = dpp_f<kQuadBcast[3]>(nf); cqv[3] = dpp_f<kQuadBcast[3]>(cq);

  f4x ae, ao;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    ae[hh] = st.acc_e[hh];
    ao[hh] = st.acc_o[hh];
  }
  // nibble masks in SGPRs and fp16 magics in VGPRs, opaque to constant
  // folding, so that each code pair is one v_and_or_b32
  uint32_t m_lo, m_hi, mg1024, mg64;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(m_lo));
  asm("s_mov_b32 %0, 0xf000f0" : "=s"(m_hi));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(mg1024));
  asm("v_mov_b32 %0, 0x54005400" : "=v"(mg64));
  uint16_t *psw = reinterpret_cast<uint16_t *>(&sm.ps[wave][0]);   // [head][group][16 tokens]
  const uint4 *pws = reinterpret_cast<const uint4 *>(psw + (hq * 4 + row) * 16);
  // one wave step over chunk c held in `cur`
  auto step = [&](const uint32_t c, const Int4Loads<D> &cur) {
    // ---- q . c of the 4 heads over this lane's (token, group)
    const uint32_t w[4] = {cur.kc.x, cur.kc.y, cur.kc.z, cur.kc.w};
    f4x d = nofv;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      // plain expressions (v_and_or_b32 with the registers above), not
      // inline asm: the compiler must see these vector writes to keep the
      // wait states before the MFMA that reads them
      const uint32_t w8 = w[ww] >> 8;
      const uint32_t x0 = (w[ww] & m_lo) | mg1024;   // channels 8ww, 8ww + 4
      const uint32_t x1 = (w[ww] & m_hi) | mg64;     // 8ww + 1, 8ww + 5
      const uint32_t x2 = (w8 & m_lo) | mg1024;      // 8ww + 2, 8ww + 6
      const uint32_t x3 = (w8 & m_hi) | mg64;        // 8ww + 3, 8ww + 7
      d = mfma4x4(qa[ww][0], qa[ww][1], x0, x1, d);
      d = mfma4x4(qa[ww][2], qa[ww][3], x2, x3, d);
    }
    // scaled group partials: cs (s q.c + z sum q) = (cs s) q.c + (cs sum q) z
    const float ssc = lo_f16(cur.ks) * P.cs;
    const float zk = hi_f16(cur.ks);
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = fmaf(ssc, d[i], cqv[i] * zk);
    // sum over the 4 groups: lane (t, h) ends with head h
    const float lgv = swap16_sum(swap32_sum(part[0], part[2]), swap32_sum(part[1], part[3]));
    const bool live = (t < n - c * SLOTS) && !((cur.bits >> bitpos) & 1u);
    const float lg = live ? lgv : kNegInf;

    if (__builtin_expect(__ballot(lg > mown) != 0, 0)) {
      // slow path: new wave max of head `row`; rescale every running quantity
      const float mn = fmaxf(mown, row16_max(lg));
      const float alpha = fast_exp2(mown - mn);          // of head `row`
      mown = mn;
      lown *= alpha;
      const float a0 = readlane_f(alpha, 0), a1 = readlane_f(alpha, 16);
      const float a2 = readlane_f(alpha, 32), a3 = readlane_f(alpha, 48);
      zl[0] *= a0; ae[0] *= a0; ao[0] *= a0;
      zl[1] *= a1; ae[1] *= a1; ao[1] *= a1;
      zl[2] *= a2; ae[2] *= a2; ao[2] *= a2;
      zl[3] *= a3; ae[3] *= a3; ao[3] *= a3;
    }
    const float p = fast_exp2(lg - mown);
    lown += p;
    // the 4 heads' p of token t in every row: after the 32-swap x holds the
    // p of row r % 2 and y that of row 2 + r % 2; the 16-swaps spread each
    float ph[4];
    float x = p, y = p;
    permlane32_swap(x, y);
    ph[0] = x; ph[1] = x;
    permlane16_swap(ph[0], ph[1]);
    ph[2] = y; ph[3] = y;
    permlane16_swap(ph[2], ph[3]);
    // V scale and the zero point of the centred codes, z + 8 s, of group
    // `row`; zero for masked tokens (their planes may hold anything)
    const uint32_t vsw = live ? cur.vs : 0u;
    const float sv = lo_f16(vsw);
    const float zv = fmaf(8.f, sv, hi_f16(vsw));
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) zl[hh] = fmaf(ph[hh], zv, zl[hh]);
    const uint32_t w01 = pack_f16_rne(ph[0] * sv, ph[1] * sv), w23 = pack_f16_rne(ph[2] * sv, ph[3] * sv);
    psw[(0 * 4 + row) * 16 + t] = static_cast<uint16_t>(w01);
    psw[(1 * 4 + row) * 16 + t] = static_cast<uint16_t>(w01 >> 16);
    psw[(2 * 4 + row) * 16 + t] = static_cast<uint16_t>(w23);
    psw[(3 * 4 + row) * 16 + t] = static_cast<uint16_t>(w23 >> 16);
    wave_sync();

    // ---- p . v (v never dequantized: sum (p s)(c - 8), zero point later)
    const uint32_t vw[4] = {cur.vc.x, cur.vc.y, cur.vc.z, cur.vc.w};
    uint32_t e[8], o[8];
    unpack_v_tile(vw, vmagic, e, o);
    const uint4 pa = pws[0], pb = pws[1];     // head hq, group row, tokens 0..7 / 8..15
    ae = mfma4x4(pa.x, pa.y, e[0], e[1], ae);
    ao = mfma4x4(pa.x, pa.y, o[0], o[1], ao);
    ae = mfma4x4(pa.z, pa.w, e[2], e[3], ae);
    ao = mfma4x4(pa.z, pa.w, o[2], o[3], ao);
    ae = mfma4x4(pb.x, pb.y, e[4], e[5], ae);
    ao = mfma4x4(pb.x, pb.y, o[4], o[5], ao);
    ae = mfma4x4(pb.z, pb.w, e[6], e[7], ae);
    ao = mfma4x4(pb.z, pb.w, o[6], o[7], ao);
  };
  // full groups of NPF steps: every refill is issued unconditionally (past
  // the split the buffer loads return 0), so each wait for the oldest ring
  // entry is a fixed count on every path into the loop
  uint32_t cb = wave;
  for (; cb + (NPF - 1) * kWaves < nsteps; cb += NPF * kWaves) {
#pragma unroll
    for (int jr = 0; jr < NPF; ++jr) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
      issue(cb + jr * kWaves + NPF * kWaves, ring[jr]);
    }
  }
  // the last NPF - 1 steps at most
#pragma unroll
  for (int jr = 0; jr < NPF - 1; ++jr)
    if (cb + jr * kWaves < nsteps) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
    }

  // ---- per-(head, group) zero-point sums, folded into the accumulators;
  // the softmax state of head hh lives in row hh
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const float z = row16_sum(zl[hh]);
    if (t == 0) sm.zo[wave][hh][row] = z;
  }
  const float lsum = row16_sum(lown);                   // head `row`, over the tokens
  wave_sync();
  const int gp = lane >> 4;                              // group of channels 2 lane, 2 lane + 1
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const float z = sm.zo[wave][hh][gp];
    st.acc_e[hh] = ae[hh] + z;
    st.acc_o[hh] = ao[hh] * 0.0625f + z;
    st.m[hh] = readlane_f(mown, 16 * hh);
    st.l[hh] = readlane_f(lsum, 16 * hh);
  }
}

// ---------------------------------------------------------------- 16-bit pass
// Element offset of row rr of the 16-bit list (VL rows first, then the window
// in position order), clamped to the last valid row; rows past r1 are masked
// by the caller.
template <int D>
__device__ __forceinline__ int64_t fp_row(const DecodeParams &P, int64_t head, int64_t rr,
                                          int64_t r1, bool *in_vl) {
  rr = rr < r1 ? rr : r1 - 1;
  *in_vl = rr < P.k;
  if (rr < P.k) return (head * P.k + rr) * D;
  int wi = P.win_offset + static_cast<int>(rr - P.k);     // < win_cap + W <= 2 win_cap
  wi -= (wi >= P.win_cap) ? P.win_cap : 0;
  return (head * P.win_cap + wi) * D;
}

template <int HT>
struct FpLoads {
  static constexpr int KW = (HT == HQ_F32) ? 32 : 16;   // dwords of 32 K channels
  static constexpr int VW = (HT == HQ_F32) ? 2 : 1;     // dwords of one V channel pair
  uint32_t k[KW];
  uint32_t v[16 * VW];
};

template <int D, int HB, int HT>
__device__ void fp_split(const DecodeParams &P, SharedMem &sm, int b, int h, int i0, int64_t r0,
                         int64_t r1, WaveState<HB> &st) {
  constexpr int LPT = D / 32;
  constexpr int SLOTS = 64 / LPT;
  constexpr int CP = D / 2;
  constexpr int EB = (HT == HQ_F32) ? 4 : 2;
  using L = FpLoads<HT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int slot = lane / LPT;
  const int g = lane % LPT;
  const int cp = lane % CP;
  const int sub = lane / CP;
  const int64_t head = static_cast<int64_t>(b) * P.Hkv + h;
  const uint8_t *vlk = static_cast<const uint8_t *>(P.vl_k);
  const uint8_t *vlv = static_cast<const uint8_t *>(P.vl_v);
  const uint8_t *wk = static_cast<const uint8_t *>(P.win_k);
  const uint8_t *wv = static_cast<const uint8_t *>(P.win_v);

  // natural query pairs (q[2i], q[2i+1]) or fp32 values for this lane's group
  uint32_t qn[HB][16];
  float qf[HB][32];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const int64_t qoff = (static_cast<int64_t>(b) * P.Hq + i0 + hh) * D + g * 32;
    if constexpr (HT == HQ_F32) {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(P.q) + qoff);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = p[i];
        qf[hh][4 * i] = f.x; qf[hh][4 * i + 1] = f.y; qf[hh][4 * i + 2] = f.z; qf[hh][4 * i + 3] = f.w;
      }
    } else {
      load_q32<HT>(P.q, qoff, qn[hh]);
    }
  }
  float zl[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) zl[hh] = 0.f;

  // every load of one wave step, issued together (addresses clamped to valid rows)
  auto issue = [&](int64_t c, L &ld) {
    const int64_t f0 = r0 + c * SLOTS;
    bool in_vl;
    const int64_t ko = fp_row<D>(P, head, f0 + slot, r1, &in_vl) + g * 32;
    const uint4 *kp = reinterpret_cast<const uint4 *>((in_vl ? vlk : wk) + ko * EB);
#pragma unroll
    for (int i = 0; i < L::KW / 4; ++i) {
      const uint4 u = kp[i];
      ld.k[4 * i] = u.x; ld.k[4 * i + 1] = u.y; ld.k[4 * i + 2] = u.z; ld.k[4 * i + 3] = u.w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bool vin;
      const int64_t vo = fp_row<D>(P, head, f0 + 16 * sub + r, r1, &vin) + 2 * cp;
      const uint8_t *vb = (vin ? vlv : wv) + vo * EB;
      if constexpr (HT == HQ_F32) {
        const uint2 u = *reinterpret_cast<const uint2 *>(vb);
        ld.v[2 * r] = u.x;
        ld.v[2 * r + 1] = u.y;
      } else {
        ld.v[r] = *reinterpret_cast<const uint32_t *>(vb);
      }
    }
  };

  const int64_t nsteps = (r1 - r0 + SLOTS - 1) / SLOTS;
  L cur, nxt;
  // row indices are clamped to the split, so every issue is in bounds and
  // needs no condition
  issue(wave, cur);
  for (int64_t c = wave; c < nsteps; c += kWaves) {
    prio_by_remaining(static_cast<uint32_t>(c), static_cast<uint32_t>(nsteps));
    issue(c + kWaves, nxt);
    const int64_t f0 = r0 + c * SLOTS;
    const bool tv = f0 + slot < r1;
    float part[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) part[hh] = 0.f;
    if constexpr (HT == HQ_F32) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float kv = __uint_as_float(cur.k[e]);
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) part[hh] = fmaf(qf[hh][e], kv, part[hh]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) part[hh] = dot2_q<HT>(qn[hh][e], cur.k[e], part[hh]);
    }
    float lg[HB];
    bool exceed = false;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float v = token_sum<LPT>(part[hh]) * P.cs;
      lg[hh] = tv ? v : kNegInf;
      exceed |= lg[hh] > st.m[hh];
    }
    if (__ballot(exceed)) raise_max<HB, LPT>(lg, st, zl);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float mu = (st.m[hh] == kNegInf) ? 0.f : st.m[hh];
      const float p = fast_exp2(lg[hh] - mu);
      st.l[hh] += p;
      if (g == 0) sm.p[wave][hh * 32 + slot] = p;
    }
    wave_sync();
    // lanes: channel pair cp over the 16 rows of sub-tile `sub` (p = 0 past r1)
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float4 *pp = reinterpret_cast<const float4 *>(&sm.p[wave][hh * 32 + 16 * sub]);
      float pr[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = pp[i];
        pr[4 * i] = f.x; pr[4 * i + 1] = f.y; pr[4 * i + 2] = f.z; pr[4 * i + 3] = f.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v0, v1;
        if constexpr (HT == HQ_F32) {
          v0 = __uint_as_float(cur.v[2 * r]);
          v1 = __uint_as_float(cur.v[2 * r + 1]);
        } else {
          v0 = half_bits_to_f32<HT>(cur.v[r] & 0xFFFFu);
          v1 = half_bits_to_f32<HT>(cur.v[r] >> 16);
        }
        st.acc_e[hh] = fmaf(pr[r], v0, st.acc_e[hh]);
        st.acc_o[hh] = fmaf(pr[r], v1, st.acc_o[hh]);
      }
    }
    wave_sync();
    cur = nxt;
  }
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    if constexpr (CP < 64) {
      st.acc_e[hh] += shfl_xor_f(st.acc_e[hh], 32);
      st.acc_o[hh] += shfl_xor_f(st.acc_o[hh], 32);
    }
    st.l[hh] = xor_sum<1>(st.l[hh]) * (1.0f / LPT);
  }
}

// ---------------------------------------------------------------- 16-bit pass, D = 128, 4 heads
// Specialisation of the 16-bit pass for head_dim 128, a chunk of 4 query
// heads and 16-bit rows, on the matrix cores with the lane layout of the
// INT4 pass (v_mfma_f32_4x4x4_16b_bf16 or _f16, sixteen 4x4x4 blocks). A
// split holds either VL rows (a contiguous block of vl_k / vl_v) or window
// rows (the ring), never both, so the chunk type is wave-uniform.
//  * Q . K: lane (token t = lane % 16, group g = lane / 16) loads the 32
//    channels of group g of its row (64 bytes) and is column t of block
//    4 g + t / 4; its A row is head lane % 4's query channels of group g in
//    the rows' own 16-bit type. MFMA j covers channels 4 j .. 4 j + 3 of the
//    group, eight of them the whole group; the permlane sums of the INT4
//    pass then give lane (t, h = lane / 16) the logit of head h for token t.
//  * Softmax as in the INT4 pass (one exponential per lane).
//  * P . V: the four heads' p (fp16, relative rounding 2^-12, as the INT4
//    pass's p s) go through LDS in the INT4 pass's layout; lane cp loads
//    channel pair cp of the chunk's 16 rows (one dword per row) and turns
//    them into fp16 token pairs (bf16 values convert exactly for magnitudes
//    in [2^-14, 65504]; smaller ones round to the fp16 subnormal grid,
//    absolute error below 2^-25), the B operand of the INT4 pass's P . V
//    MFMAs. No zero point: the rows are the values themselves.
struct FpRing {
  u32x4 k[4];                 // 32 key channels of this lane's (row, group)
  uint32_t v[16];             // value channel pair cp of the chunk's 16 rows
};

template <int QT>
__device__ __forceinline__ f4x mfma4x4_16b(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f4x c) {
  if constexpr (QT == HQ_BF16) {
    typedef short s4x __attribute__((ext_vector_type(4)));
    const u2x a = {a0, a1}, bb = {b0, b1};
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s4x, a), __builtin_bit_cast(s4x, bb), c, 0, 0,
                                                   0);
  } else {
    return mfma4x4(a0, a1, b0, b1, c);
  }
}
// two 16-bit values (low halves of x and y, or high halves) as an fp16 pair
template <int QT, bool HI>
__device__ __forceinline__ uint32_t pair_f16(uint32_t x, uint32_t y) {
  if constexpr (QT == HQ_F16) {
    return HI ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
  } else {
    const float fx = __uint_as_float(HI ? (x & 0xFFFF0000u) : (x << 16));
    const float fy = __uint_as_float(HI ? (y & 0xFFFF0000u) : (y << 16));
    return pack_f16_rne(fx, fy);
  }
}

template <int QT, bool WIN>
__device__ void fp_rows_d128_g4(const DecodeParams &P, SharedMem &sm, int b, int h, int i0,
                                int64_t r0, int64_t r1, WaveState<4> &st) {
  constexpr int D = 128, SLOTS = 16, RB = D * 2;   // RB: bytes per row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;             // row of the chunk
  const int row = lane >> 4;           // key group (loads, Q . K), head (softmax)
  const int hq = lane & 3;             // head of this lane's A row
  const int64_t head = static_cast<int64_t>(b) * P.Hkv + h;

  // query channels of head hq, group `row`, natural pairs (2c, 2c + 1)
  uint32_t qw[16];
  load_q32<QT>(P.q, (static_cast<int64_t>(b) * P.Hq + i0 + hq) * D + row * 32, qw);
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t n = static_cast<uint32_t>(r1 - r0);
  const uint8_t *kbase, *vbase;
  uint32_t kbytes;
  int wrow0 = 0;
  if constexpr (!WIN) {
    // rows [r0, r1) of the head's VL block; views past r1 read as 0
    kbase = static_cast<const uint8_t *>(P.vl_k) + (head * P.k + r0) * RB;
    vbase = static_cast<const uint8_t *>(P.vl_v) + (head * P.k + r0) * RB;
    kbytes = n * RB;
  } else {
    // the head's ring of win_cap rows; list row k + w is ring row (win_offset + w) mod win_cap
    kbase = static_cast<const uint8_t *>(P.win_k) + head * P.win_cap * RB;
    vbase = static_cast<const uint8_t *>(P.win_v) + head * P.win_cap * RB;
    kbytes = static_cast<uint32_t>(P.win_cap) * RB;
    wrow0 = P.win_offset + static_cast<int>(r0 - P.k);      // ring row of the split's first row, < win_cap + W
  }
  auto ring_row = [&](int w) {                                // w < win_cap + 2 W <= 3 win_cap
    w -= (w >= P.win_cap) ? P.win_cap : 0;
    w -= (w >= P.win_cap) ? P.win_cap : 0;
    return w;
  };
  auto issue = [&](uint32_t c, FpRing &L) {
    const uint32_t f = c * SLOTS;                              // first row of the chunk in the split
    if constexpr (!WIN) {
      const __amdgpu_buffer_rsrc_t rk = view(kbase, kbytes, f * RB);
      const __amdgpu_buffer_rsrc_t rv = view(vbase, kbytes, f * RB);
      const uint32_t ko = t * RB + row * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) L.k[i] = bload16(rk, ko + 16 * i);
#pragma unroll
      for (int r = 0; r < 16; ++r) L.v[r] = bload4(rv, lane * 4 + r * RB);
    } else {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, kbytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, kbytes);
      const uint32_t ko = static_cast<uint32_t>(ring_row(wrow0 + static_cast<int>(f) + t)) * RB + row * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) L.k[i] = bload16(rk, ko + 16 * i);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        L.v[r] = bload4(rv, lane * 4 + static_cast<uint32_t>(ring_row(wrow0 + static_cast<int>(f) + r)) * RB);
    }
  };

  // no prefetch ring: each wave issues the next chunk's loads after its
  // current chunk (the other waves on the SIMD cover the wait)
  constexpr int NPF = 1;
  const uint32_t nsteps = (n + SLOTS - 1) / SLOTS;
  FpRing ring[NPF];
#pragma unroll
  for (int jr = 0; jr < NPF; ++jr) {
    issue(wave + jr * kWaves, ring[jr]);
    __builtin_amdgcn_sched_barrier(0);
  }
  float mown = -__FLT_MAX__;            // running max of head `row` (finite: see the INT4 pass)
  float lown = 0.f;
  f4x ae = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
  uint16_t *psw = reinterpret_cast<uint16_t *>(&sm.ps[wave][0]);   // [head][group][16 rows]
  const uint4 *pws = reinterpret_cast<const uint4 *>(psw + (hq * 4 + row) * 16);

  auto step = [&](const uint32_t c, const FpRing &cur) {
    // ---- q . k of the 4 heads over this lane's (row, group)
    const uint32_t kw[16] = {cur.k[0].x, cur.k[0].y, cur.k[0].z, cur.k[0].w,
                             cur.k[1].x, cur.k[1].y, cur.k[1].z, cur.k[1].w,
                             cur.k[2].x, cur.k[2].y, cur.k[2].z, cur.k[2].w,
                             cur.k[3].x, cur.k[3].y, cur.k[3].z, cur.k[3].w};
    f4x d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) d = mfma4x4_16b<QT>(qw[2 * j], qw[2 * j + 1], kw[2 * j], kw[2 * j + 1], d);
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = d[i] * P.cs;
    const float lgv = swap16_sum(swap32_sum(part[0], part[2]), swap32_sum(part[1], part[3]));
    const bool live = t < n - c * SLOTS;
    const float lg = live ? lgv : kNegInf;
    if (__builtin_expect(__ballot(lg > mown) != 0, 0)) {
      const float mn = fmaxf(mown, row16_max(lg));
      const float alpha = fast_exp2(mown - mn);          // of head `row`
      mown = mn;
      lown *= alpha;
      const float a0 = readlane_f(alpha, 0), a1 = readlane_f(alpha, 16);
      const float a2 = readlane_f(alpha, 32), a3 = readlane_f(alpha, 48);
      ae[0] *= a0; ao[0] *= a0;
      ae[1] *= a1; ao[1] *= a1;
      ae[2] *= a2; ao[2] *= a2;
      ae[3] *= a3; ao[3] *= a3;
    }
    const float p = fast_exp2(lg - mown);
    lown += p;
    float ph[4];
    float x = p, y = p;
    permlane32_swap(x, y);
    ph[0] = x; ph[1] = x;
    permlane16_swap(ph[0], ph[1]);
    ph[2] = y; ph[3] = y;
    permlane16_swap(ph[2], ph[3]);
    const uint32_t w01 = pack_f16_rne(ph[0], ph[1]), w23 = pack_f16_rne(ph[2], ph[3]);
    psw[(0 * 4 + row) * 16 + t] = static_cast<uint16_t>(w01);
    psw[(1 * 4 + row) * 16 + t] = static_cast<uint16_t>(w01 >> 16);
    psw[(2 * 4 + row) * 16 + t] = static_cast<uint16_t>(w23);
    psw[(3 * 4 + row) * 16 + t] = static_cast<uint16_t>(w23 >> 16);
    wave_sync();

    // ---- p . v: fp16 token pairs of this lane's channel pair
    uint32_t e[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = pair_f16<QT, false>(cur.v[2 * i], cur.v[2 * i + 1]);
      o[i] = pair_f16<QT, true>(cur.v[2 * i], cur.v[2 * i + 1]);
    }
    const uint4 pa = pws[0], pb = pws[1];     // head hq, tokens 0..7 / 8..15
    ae = mfma4x4(pa.x, pa.y, e[0], e[1], ae);
    ao = mfma4x4(pa.x, pa.y, o[0], o[1], ao);
    ae = mfma4x4(pa.z, pa.w, e[2], e[3], ae);
    ao = mfma4x4(pa.z, pa.w, o[2], o[3], ao);
    ae = mfma4x4(pb.x, pb.y, e[4], e[5], ae);
    ao = mfma4x4(pb.x, pb.y, o[4], o[5], ao);
    ae = mfma4x4(pb.z, pb.w, e[6], e[7], ae);
    ao = mfma4x4(pb.z, pb.w, o[6], o[7], ao);
    wave_sync();
  };
  uint32_t cb = wave;
  for (; cb + (NPF - 1) * kWaves < nsteps; cb += NPF * kWaves) {
#pragma unroll
    for (int jr = 0; jr < NPF; ++jr) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
      issue(cb + jr * kWaves + NPF * kWaves, ring[jr]);
    }
  }
#pragma unroll
  for (int jr = 0; jr < NPF - 1; ++jr)
    if (cb + jr * kWaves < nsteps) {
      prio_by_remaining(cb + jr * kWaves, nsteps);
      step(cb + jr * kWaves, ring[jr]);
    }

  const float lsum = row16_sum(lown);                   // head `row`, over the rows
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    st.acc_e[hh] = ae[hh];
    st.acc_o[hh] = ao[hh];
    st.m[hh] = readlane_f(mown, 16 * hh);
    st.l[hh] = readlane_f(lsum, 16 * hh);
  }
}

// ---------------------------------------------------------------- the kernel
template <int D, int HB, int QT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams P) {
  __shared__ SharedMem sm;
  constexpr int CP = D / 2;
  // XCD-aware numbering: hardware block id -> (xcd, index on that xcd)
  const int hw = blockIdx.x;
  const int lin = (hw % kNumXcd) * P.blocks_per_xcd + hw / kNumXcd;
  if (lin >= P.blocks_used) return;
  // the head chunks of one KV head are adjacent for each split, so they
  // run together on one XCD and read each KV tile from HBM once (the other
  // chunks' reads hit that XCD's L2)
  int hc, split, bh;
  if (P.upx > 0) {
    // each XCD holds whole units: it runs all their INT4 splits first, then
    // the VL splits, then the window splits, so that the shorter 16-bit
    // blocks are the last ones dispatched and fill the tail
    const int x = lin / P.blocks_per_xcd;
    const int li = lin - x * P.blocks_per_xcd;
    const int nq4 = P.upx * P.nhc * P.S_q, nvl = P.upx * P.nhc * P.S_vl;
    int r, s0, ns;
    if (li < nq4) {
      r = li, s0 = 0, ns = P.S_q;
    } else if (li < nq4 + nvl) {
      r = li - nq4, s0 = P.S_q, ns = P.S_vl;
    } else {
      r = li - nq4 - nvl, s0 = P.S_q + P.S_vl, ns = P.S_win;
    }
    hc = r % P.nhc;
    split = s0 + (r / P.nhc) % ns;
    bh = x * P.upx + r / (P.nhc * ns);
  } else {
    hc = lin % P.nhc;
    split = (lin / P.nhc) % P.S;
    bh = lin / (P.nhc * P.S);
  }
  const int h = bh % P.Hkv;
  const int b = bh / P.Hkv;
  const int i0 = h * P.G + hc * HB;           // first query head of this block

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)

  WaveState<HB> st;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    st.m[hh] = kNegInf;
    st.l[hh] = 0.f;
    st.acc_e[hh] = 0.f;
    st.acc_o[hh] = 0.f;
  }
  if (split < P.S_q) {
    const int64_t r0 = static_cast<int64_t>(split) * P.len_q;
    const int64_t r1 = r0 + P.len_q < P.nq ? r0 + P.len_q : P.nq;
    if constexpr (D == 128 && HB == 4 && QT != HQ_F32)
      int4_split_d128_g4<QT>(P, sm, b, h, i0, r0, r1, st);
    else
      int4_split<D, HB, QT>(P, sm, b, h, i0, r0, r1, st);
  } else {
    // rows [r0, r1) of the 16-bit list (VL rows 0..k-1, then the W window
    // rows); a split lies entirely in one of the two parts
    int64_t r0, r1;
    const bool win = split >= P.S_q + P.S_vl;
    if (!win) {
      r0 = static_cast<int64_t>(split - P.S_q) * P.len_vl;
      r1 = r0 + P.len_vl < P.k ? r0 + P.len_vl : P.k;
    } else {
      r0 = P.k + static_cast<int64_t>(split - P.S_q - P.S_vl) * P.len_win;
      r1 = r0 + P.len_win < static_cast<int64_t>(P.k) + P.W ? r0 + P.len_win : static_cast<int64_t>(P.k) + P.W;
    }
    if constexpr (D == 128 && HB == 4 && QT != HQ_F32) {
      if (win) fp_rows_d128_g4<QT, true>(P, sm, b, h, i0, r0, r1, st);
      else fp_rows_d128_g4<QT, false>(P, sm, b, h, i0, r0, r1, st);
    } else {
      fp_split<D, HB, QT>(P, sm, b, h, i0, r0, r1, st);
    }
  }

  // ---- combine the 4 waves
  if (lane < CP) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      sm.bo[wave][hh][2 * lane] = st.acc_e[hh];
      sm.bo[wave][hh][2 * lane + 1] = st.acc_o[hh];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      sm.bm[wave][hh] = st.m[hh];
      sm.bl[wave][hh] = st.l[hh];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < HB * D; e += kThreads) {
    const int hh = e / D;
    const int d = e % D;
    float mb = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, sm.bm[w][hh]);
    const float mu = (mb == kNegInf) ? 0.f : mb;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm.bm[w][hh] - mu);
      o = fmaf(f, sm.bo[w][hh][d], o);
      l = fmaf(f, sm.bl[w][hh], l);
    }
    const int64_t pidx = (static_cast<int64_t>(b) * P.Hq + i0 + hh) * P.S + split;
    P.part_o[pidx * D + d] = o;
    if (d == 0) P.part_ml[pidx] = make_float2(mb, l);
  }

}

// ---------------------------------------------------------------- split merge
// One block per (unit, query head, 32-channel slice): out = sum_s w_s o_s / L
// with w_s = 2^(m_s - m*), m* = max_s m_s and L = sum_s w_s l_s; lse = (m* +
// log2 L) ln 2. A kernel of its own: the launch boundary makes every split's
// partial visible without device-scope fences inside the split kernel. All
// loads are issued first. Each wave finds m* and L over all splits by itself
// (the same values in the same lanes and the same reduction order, so every
// wave gets the same numbers); thread t weights float4 t % 8 of the slice for
// the splits t / 8, t / 8 + 32, ..., and the 32 split groups are summed in a
// fixed order, so the result is deterministic.
constexpr int kMergeSlice = 32;
constexpr bool kTypeMajor = true;   // dispatch each XCD's INT4 splits before its 16-bit ones

// Per-step upkeep of hq_decode_step. It runs in the merge launch, after every
// split has read the cache, so writing INT4 row T - W (outside this step's
// INT4 range [0, T - W)) cannot race with them.
//  * the first up_q blocks: q [B][Hq][D] into slot ring_slot of q_ring, one
//    16-byte chunk per thread;
//  * the next blocks (if evict): the window's oldest row (position T - W, ring
//    row win_offset) of every (b, KV head) packed like hq_quantize_kv_pair:
//    four lanes (a DPP quad) per 32-channel group, K in rows, V in TILE16.
template <int D, int QT>
__device__ void upkeep(const DecodeParams &P, int ub) {
  constexpr int EB = QT == HQ_F32 ? 4 : 2;
  constexpr int NG = D / 32;
  if (ub < P.up_q) {
    constexpr int CH = D * EB / 16;                         // 16-byte chunks per q row
    const int c = ub * kThreads + static_cast<int>(threadIdx.x);
    if (c < P.B * P.Hq * CH) {
      const int r = c / CH, cc = c % CH;
      const uint4 v = reinterpret_cast<const uint4 *>(P.q)[c];
      reinterpret_cast<uint4 *>(P.q_ring + (static_cast<int64_t>(r) * P.R + P.ring_slot) * (D * EB))[cc] = v;
    }
    return;
  }
  const uint32_t per = 4u * static_cast<uint32_t>(P.B * P.Hkv) * NG;    // threads per tensor
  const uint32_t gid = static_cast<uint32_t>(ub - P.up_q) * kThreads + threadIdx.x;
  if (gid >= 2u * per) return;                             // whole quads: per is a multiple of 4
  const bool is_v = gid >= per;
  const uint32_t lg = is_v ? gid - per : gid;
  const int qq = static_cast<int>(lg & 3u);
  const uint32_t item = lg >> 2;
  const int g = static_cast<int>(item % NG);
  const int64_t hd = item / NG;                             // b * Hkv + h
  const void *src = is_v ? P.win_v : P.win_k;
  float v[8];
  load8<QT>(src, (hd * P.win_cap + P.win_offset) * D + g * 32 + qq * 8, v);
  _Float16 s16, z16;
  const uint32_t packed = encode_quarter(v, s16, z16);
  const int64_t row = P.nq;                                 // position T - W
  const int64_t head_row = hd * P.t_cap + row;
  if (!is_v) {
    reinterpret_cast<uint32_t *>(P.ek_codes + head_row * (D / 2) + g * 16)[qq] = packed;
  } else {
    // tile row / 16 of the head; byte (j, slot16(row % 16)), each run of 4
    // rows stored in the order 0, 2, 1, 3
    const int64_t tile = hd * (P.t_cap / 16) + row / 16;
    const int r16 = static_cast<int>(row % 16);
    const int slot16 = (r16 & ~3) | ((r16 & 1) << 1) | ((r16 >> 1) & 1);
    uint8_t *base = P.ev_codes + tile * (D / 2) * 16 + slot16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      base[(g * 16 + qq * 4 + jj) * 16] = static_cast<uint8_t>((packed >> (8 * jj)) & 0xFFu);
  }
  if (qq == 0) {
    const uint32_t szw = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
    (is_v ? P.ev_sz : P.ek_sz)[head_row * NG + g] = szw;
  }
}

template <int D, int HB, int QT>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams P) {
  // XCD-aware numbering as in the split kernel: merge block m runs on the XCD
  // whose L2 the unit's splits wrote their partials through
  const int hw = blockIdx.x;
  const int mgrid = kNumXcd * P.merge_per_xcd;
  if (hw >= mgrid) {                                         // block-uniform
    upkeep<D, QT>(P, hw - mgrid);
    return;
  }
  const int mb = (hw % kNumXcd) * P.merge_per_xcd + hw / kNumXcd;
  if (mb >= P.merge_blocks) return;
  constexpr int NSL = D / kMergeSlice;            // slices per head
  constexpr int F4 = kMergeSlice / 4;             // float4 per slice row
  constexpr int SG = kThreads / F4;               // split groups
  constexpr int MAXO = kMaxSplits / SG;           // partial rows per thread at most
  constexpr int MAXM = kMaxSplits / 64;           // (m, l) pairs per lane at most
  static_assert(kMaxSplits % SG == 0 && kMaxSplits % 64 == 0, "split tiling");
  __shared__ float sw[kMaxSplits];
  __shared__ float4 red[SG][F4];
  const int sl = mb % NSL;
  const int qh = mb / NSL;
  const int unit = qh / HB;
  const int hh = qh % HB;
  const int hc = unit % P.nhc;
  const int bh = unit / P.nhc;
  const int h = bh % P.Hkv;
  const int b = bh / P.Hkv;
  const int64_t qi = static_cast<int64_t>(b) * P.Hq + h * P.G + hc * HB + hh;
  const int S = P.S;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int f = t % F4, sg = t / F4;
  const float4 *po = reinterpret_cast<const float4 *>(P.part_o) + qi * S * (D / 4) + sl * F4 + f;
  float4 v[MAXO];
#pragma unroll
  for (int i = 0; i < MAXO; ++i) {
    const int sp = sg + i * SG;
    v[i] = sp < S ? po[static_cast<int64_t>(sp) * (D / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float2 ml[MAXM];
#pragma unroll
  for (int i = 0; i < MAXM; ++i) {
    const int sp = lane + 64 * i;
    ml[i] = sp < S ? P.part_ml[qi * S + sp] : make_float2(kNegInf, 0.f);
  }
  float mx = ml[0].x;
#pragma unroll
  for (int i = 1; i < MAXM; ++i) mx = fmaxf(mx, ml[i].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
  const float mu = (mx == kNegInf) ? 0.f : mx;
  float lw = 0.f;
#pragma unroll
  for (int i = 0; i < MAXM; ++i) {
    const int sp = lane + 64 * i;
    const float wgt = sp < S ? fast_exp2(ml[i].x - mu) : 0.f;
    if (wave == 0 && sp < S) sw[sp] = wgt;
    lw = fmaf(wgt, ml[i].y, lw);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lw += shfl_xor_f(lw, o);
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MAXO; ++i) {
    const int sp = sg + i * SG;
    if (sp < S) {
      const float wgt = sw[sp];
      acc.x = fmaf(wgt, v[i].x, acc.x);
      acc.y = fmaf(wgt, v[i].y, acc.y);
      acc.z = fmaf(wgt, v[i].z, acc.z);
      acc.w = fmaf(wgt, v[i].w, acc.w);
    }
  }
  red[sg][f] = acc;
  __syncthreads();
  if (t < kMergeSlice) {
    const float *rf = reinterpret_cast<const float *>(&red[0][0]);
    float o = 0.f;
#pragma unroll 8
    for (int g2 = 0; g2 < SG; ++g2) o += rf[g2 * kMergeSlice + t];
    P.out[qi * D + sl * kMergeSlice + t] = o / lw;
    if (t == 0 && sl == 0 && P.lse) P.lse[qi] = (mu + log2f(lw)) * kLn2;
  }
}

// ---------------------------------------------------------------- VL bitmap
// One block per (b, h): bits[h][w] has bit t%32 of word t/32 set iff t is in
// vl_idx[h][0..k). Words are built in LDS segments of 8192 words.
constexpr int kSegWords = 8192;
__global__ __launch_bounds__(256) void vl_bitmap_kernel(const int32_t *__restrict__ idx, int k,
                                                        int64_t words, uint32_t *__restrict__ bits) {
  __shared__ uint32_t seg[kSegWords];
  const int64_t h = blockIdx.x;
  const int32_t *ih = idx + h * k;
  uint32_t *bh = bits + h * words;
  for (int64_t w0 = 0; w0 < words; w0 += kSegWords) {
    const int64_t nw = (words - w0) < kSegWords ? (words - w0) : kSegWords;
    for (int i = threadIdx.x; i < nw; i += blockDim.x) seg[i] = 0u;
    __syncthreads();
    const int64_t lo = w0 * 32, hi = (w0 + nw) * 32;
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
      const int64_t t = ih[i];
      if (t >= lo && t < hi) atomicOr(&seg[(t - lo) >> 5], 1u << ((t - lo) & 31));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nw; i += blockDim.x) bh[w0 + i] = seg[i];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- planning
struct Plan {
  int nhc, HB, units, S_q, S_vl, S_win, S;
  int64_t len_q;
  int len_vl, len_win;
  int64_t nq;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

Plan make_plan(const hq_hybrid_kv *kv, int Hq, int n_splits) {
  Plan pl{};
  const int G = Hq / kv->Hkv;
  pl.HB = G >= 4 ? 4 : G;
  pl.nhc = G / pl.HB;
  pl.units = kv->B * kv->Hkv * pl.nhc;
  const int step = 64 / (kv->D / 32);                         // positions per wave step
  const int64_t gran = static_cast<int64_t>(kWaves) * step;   // INT4 split granularity (64 or 128)
  pl.nq = kv->T - kv->W;
  // positions of the INT4 pass (none when the INT4 set is dropped)
  const int64_t nq_att = (kv->flags & HQ_KV_DROP_INT4) ? 0 : pl.nq;
  const int64_t nfp = static_cast<int64_t>(kv->k) + kv->W;
  // Splits are sized by cost, not bytes: a 16-bit row costs about twice an
  // INT4 position (fp32 P . V products and 3.2x the bytes, against the
  // unpacking of the codes).
  constexpr double kFpRowCost = 2.0;
  const double cost_q = static_cast<double>(nq_att);
  const double cost_fp = kFpRowCost * static_cast<double>(nfp);
  int S = n_splits;
  if (S <= 0) {
    // one generation of 512 blocks fills the chip; long contexts get six,
    // so that blocks finishing early are replaced and the tail stays short
    // (at 16 x 128K tokens, 8 KV heads: 533 us with 2048 blocks, 503 with
    // 3072, 505 with 4096)
    const double steps_per_wave = (cost_q + cost_fp) / step * pl.units / (512.0 * kWaves);
    const int target_blocks = steps_per_wave >= 128.0 ? 3072 : 512;
    S = static_cast<int>(ceil_div(target_blocks, pl.units));
    // at least ~4 wave steps of work per wave
    const int64_t max_s = ceil_div(nq_att + nfp, 16LL * step);
    if (S > max_s) S = static_cast<int>(max_s > 0 ? max_s : 1);
    if (S > kMaxSplits) S = kMaxSplits;
    if (S < 1) S = 1;
  }
  // 16-bit splits: the VL rows and the window rows are rounded up each on
  // their own, so that no 16-bit split costs more than an average split (a
  // long VL split would otherwise be the launch's tail)
  const double avg = (cost_q + cost_fp) / S;
  int s_vl = 0, s_win = 0;
  if (kv->k > 0) {
    s_vl = static_cast<int>(std::ceil(kFpRowCost * kv->k / avg - 1e-9));
    const int64_t mx = ceil_div(kv->k, step);
    if (s_vl > mx) s_vl = static_cast<int>(mx);
    if (s_vl < 1) s_vl = 1;
  }
  if (kv->W > 0) {
    s_win = static_cast<int>(std::ceil(kFpRowCost * kv->W / avg - 1e-9));
    const int64_t mx = ceil_div(kv->W, step);
    if (s_win > mx) s_win = static_cast<int>(mx);
    if (s_win < 1) s_win = 1;
  }
  int s_q = 0;
  if (nq_att > 0) {
    s_q = S - s_vl - s_win;
    if (s_q < 1) s_q = 1;
    // the VL bitmap and the ranges: at most 2^20 positions per split
    const int64_t mn = ceil_div(nq_att, 1LL << 20);
    if (s_q < mn) s_q = static_cast<int>(mn);
    const int64_t mx = ceil_div(nq_att, gran);
    if (s_q > mx) s_q = static_cast<int>(mx);
  }
  // INT4 splits start at multiples of gran (a multiple of 64): the kernel
  // reads the VL bits of a chunk from one aligned bitmap word
  pl.len_q = s_q > 0 ? ceil_div(ceil_div(nq_att, s_q), gran) * gran : 0;
  pl.S_q = s_q > 0 ? static_cast<int>(ceil_div(nq_att, pl.len_q)) : 0;
  pl.len_vl = s_vl > 0 ? static_cast<int>(ceil_div(ceil_div(kv->k, s_vl), step) * step) : 0;
  pl.S_vl = s_vl > 0 ? static_cast<int>(ceil_div(kv->k, pl.len_vl)) : 0;
  pl.len_win = s_win > 0 ? static_cast<int>(ceil_div(ceil_div(kv->W, s_win), step) * step) : 0;
  pl.S_win = s_win > 0 ? static_cast<int>(ceil_div(kv->W, pl.len_win)) : 0;
  pl.S = pl.S_q + pl.S_vl + pl.S_win;
  return pl;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t ml, o, total;
};
WsLayout ws_layout(const hq_hybrid_kv *kv, int Hq, const Plan &pl) {
  WsLayout L{};
  L.ml = 0;
  L.o = L.ml + align_up(static_cast<size_t>(kv->B) * Hq * pl.S * sizeof(float2), 256);
  L.total = L.o + static_cast<size_t>(kv->B) * Hq * pl.S * kv->D * sizeof(float);
  return L;
}

// rows of the window ring: win_cap, or W when win_cap is 0
int ring_rows(const hq_hybrid_kv *kv) { return kv->win_cap > 0 ? kv->win_cap : kv->W; }

hq_status validate(const void *q, int q_dtype, int Hq, const hq_hybrid_kv *kv, float *out) {
  if (!kv) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: null descriptor");
  if (kv->B < 1 || kv->Hkv < 1 || Hq < 1) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: B, Hkv, Hq must be >= 1");
  if (Hq % kv->Hkv) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: Hq %% Hkv != 0");
  const int G = Hq / kv->Hkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16))
    return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn: G = %d not in {1,2,4,8,16}", G);
  if (kv->D != 64 && kv->D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn: D must be 64 or 128");
  if (kv->group != 32) return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn: group must be 32");
  if (!dtype_ok(q_dtype) || !dtype_ok(kv->hp_dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: bad dtype");
  if (q_dtype != kv->hp_dtype)
    return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn: q dtype must equal the 16-bit rows' dtype");
  if (kv->T < 1) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: T must be >= 1");
  if (kv->W < 0 || kv->W > kv->T) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: need 0 <= W <= T");
  if (kv->k < 0 || kv->k > kv->T - kv->W) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: need 0 <= k <= T - W");
  if (kv->t_cap < kv->T - kv->W || kv->t_cap % 32 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: t_cap must be >= T - W and a multiple of 32");
  if (kv->win_cap != 0 && kv->win_cap < kv->W)
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: win_cap must be 0 or >= W");
  if (kv->W > 0 && (kv->win_offset < 0 || kv->win_offset >= ring_rows(kv)))
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: win_offset out of range");
  if (!q || !out) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: null q or out");
  if (kv->flags & ~HQ_KV_DROP_INT4) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: unknown flags");
  if (kv->T - kv->W > 0 && !(kv->flags & HQ_KV_DROP_INT4) &&
      (!kv->k_codes || !kv->v_codes || !kv->k_sz || !kv->v_sz || !kv->vl_bits))
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: null INT4 plane or VL bitmap");
  if (kv->k > 0 && (!kv->vl_k || !kv->vl_v)) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: null VL rows");
  if (kv->W > 0 && (!kv->win_k || !kv->win_v)) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: null window rows");
  // dropping the INT4 set with no VL and no window rows leaves nothing to attend to
  if ((kv->flags & HQ_KV_DROP_INT4) && kv->k == 0 && kv->W == 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: HQ_KV_DROP_INT4 with k == 0 and W == 0 is an empty softmax");
  // the scale planes and the bitmap are read as 32-bit words
  if ((reinterpret_cast<uintptr_t>(kv->k_sz) | reinterpret_cast<uintptr_t>(kv->v_sz) |
       reinterpret_cast<uintptr_t>(kv->vl_bits)) % 4)
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: k_sz, v_sz and vl_bits must be 4-byte aligned");
  const uintptr_t al = reinterpret_cast<uintptr_t>(kv->k_codes) | reinterpret_cast<uintptr_t>(kv->v_codes) |
                       reinterpret_cast<uintptr_t>(kv->vl_k) | reinterpret_cast<uintptr_t>(kv->vl_v) |
                       reinterpret_cast<uintptr_t>(kv->win_k) | reinterpret_cast<uintptr_t>(kv->win_v) |
                       reinterpret_cast<uintptr_t>(q);
  if (al % 16) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: buffers must be 16-byte aligned");
  return HQ_OK;
}

template <int D, int HB, int QT>
void launch_qt(dim3 grid, dim3 mgrid, hipStream_t st, const DecodeParams &P) {
  hipLaunchKernelGGL((decode_kernel<D, HB, QT>), grid, dim3(kThreads), 0, st, P);
  hipLaunchKernelGGL((merge_kernel<D, HB, QT>), mgrid, dim3(kThreads), 0, st, P);
}
template <int D, int HB>
void launch_hb(int qdt, dim3 grid, hipStream_t st, const DecodeParams &P) {
  const dim3 mgrid(static_cast<unsigned>(kNumXcd * P.merge_per_xcd + P.up_q) +
                   (P.evict ? static_cast<unsigned>((8 * P.B * P.Hkv * (D / 32) + kThreads - 1) / kThreads) : 0u));
  switch (qdt) {
    case HQ_F32: launch_qt<D, HB, HQ_F32>(grid, mgrid, st, P); break;
    case HQ_BF16: launch_qt<D, HB, HQ_BF16>(grid, mgrid, st, P); break;
    default: launch_qt<D, HB, HQ_F16>(grid, mgrid, st, P); break;
  }
}
template <int D>
void launch_d(int HB, int qdt, dim3 grid, hipStream_t st, const DecodeParams &P) {
  switch (HB) {
    case 1: launch_hb<D, 1>(qdt, grid, st, P); break;
    case 2: launch_hb<D, 2>(qdt, grid, st, P); break;
    default: launch_hb<D, 4>(qdt, grid, st, P); break;
  }
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" int hq_decode_auto_splits(const hq_hybrid_kv *kv, int Hq) {
  if (!kv || kv->Hkv < 1 || Hq % kv->Hkv) return 0;
  return make_plan(kv, Hq, 0).S;
}

extern "C" size_t hq_decode_workspace_size(const hq_hybrid_kv *kv, int Hq, int n_splits) {
  if (!kv || kv->Hkv < 1 || Hq < 1 || Hq % kv->Hkv || kv->T < 1 || (kv->D != 64 && kv->D != 128))
    return 0;
  const Plan pl = make_plan(kv, Hq, n_splits);
  return ws_layout(kv, Hq, pl).total;
}

namespace hq {
namespace {
struct Upkeep {
  void *q_ring = nullptr;
  int R = 0, slot = 0;
  bool evict = false;
};
hq_status decode_common(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv, float sm_scale,
                        int n_splits, float *out, float *lse, void *ws, size_t ws_bytes, const Upkeep &up,
                        void *stream) {
  const hq_status s = validate(q, q_dtype, Hq, kv, out);
  if (s != HQ_OK) return s;
  if (n_splits < 0) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: n_splits < 0");
  const Plan pl = make_plan(kv, Hq, n_splits);
  if (pl.S > kMaxSplits)
    return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn: %d splits exceed the maximum %d", pl.S, kMaxSplits);
  const WsLayout L = ws_layout(kv, Hq, pl);
  if (!ws || ws_bytes < L.total)
    return fail(HQ_ERR_WORKSPACE, "hq_decode_attn: workspace needs %zu bytes, got %zu", L.total, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: workspace must be 256-byte aligned");
  DecodeParams P{};
  P.q = q;
  P.k_codes = kv->k_codes;
  P.v_codes = kv->v_codes;
  P.k_sz = reinterpret_cast<const uint32_t *>(kv->k_sz);
  P.v_sz = reinterpret_cast<const uint32_t *>(kv->v_sz);
  P.vl_bits = kv->vl_bits;
  P.vl_k = kv->vl_k;
  P.vl_v = kv->vl_v;
  P.win_k = kv->win_k;
  P.win_v = kv->win_v;
  P.out = out;
  P.lse = lse;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  P.part_ml = reinterpret_cast<float2 *>(w8 + L.ml);
  P.part_o = reinterpret_cast<float *>(w8 + L.o);
  P.t_cap = kv->t_cap;
  P.nq = pl.nq;
  P.bits_words = kv->t_cap / 32;
  P.k = kv->k;
  P.W = kv->W;
  P.win_offset = kv->win_offset;
  P.win_cap = ring_rows(kv);
  P.B = kv->B;
  P.Hkv = kv->Hkv;
  P.Hq = Hq;
  P.G = Hq / kv->Hkv;
  P.nhc = pl.nhc;
  P.S_q = pl.S_q;
  P.S_vl = pl.S_vl;
  P.S_win = pl.S_win;
  P.S = pl.S;
  P.len_q = pl.len_q;
  P.len_vl = pl.len_vl;
  P.len_win = pl.len_win;
  P.units = pl.units;
  P.blocks_used = pl.units * pl.S;
  const int blocks = static_cast<int>(ceil_div(P.blocks_used, kNumXcd) * kNumXcd);
  P.blocks_per_xcd = blocks / kNumXcd;
  {
    const int per_unit = pl.nhc * pl.S;                     // blocks of one (b, KV head)
    P.upx = (kTypeMajor && blocks == P.blocks_used && P.blocks_per_xcd % per_unit == 0)
                ? P.blocks_per_xcd / per_unit : 0;
  }
  const float scale = sm_scale == 0.f ? 1.0f / sqrtf(static_cast<float>(kv->D)) : sm_scale;
  P.cs = scale * kLog2e;
  P.merge_blocks = pl.units * pl.HB * (kv->D / kMergeSlice);
  P.merge_per_xcd = static_cast<int>(ceil_div(P.merge_blocks, kNumXcd));
  P.up_q = up.q_ring ? static_cast<int>(ceil_div(static_cast<int64_t>(kv->B) * Hq * kv->D *
                                                    (q_dtype == HQ_F32 ? 4 : 2) / 16, kThreads))
                     : 0;
  P.q_ring = static_cast<uint8_t *>(up.q_ring);
  P.R = up.R;
  P.ring_slot = up.slot;
  P.evict = up.evict ? 1 : 0;
  P.ek_codes = const_cast<uint8_t *>(kv->k_codes);
  P.ev_codes = const_cast<uint8_t *>(kv->v_codes);
  P.ek_sz = reinterpret_cast<uint32_t *>(const_cast<uint16_t *>(kv->k_sz));
  P.ev_sz = reinterpret_cast<uint32_t *>(const_cast<uint16_t *>(kv->v_sz));
  hipStream_t st = as_stream(stream);
  if (kv->D == 128) launch_d<128>(pl.HB, q_dtype, dim3(blocks), st, P);
  else launch_d<64>(pl.HB, q_dtype, dim3(blocks), st, P);
  return HQ_OK;
}
}  // namespace
}  // namespace hq

extern "C" hq_status hq_decode_attn(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                                    float sm_scale, int n_splits, float *out, float *lse, void *ws,
                                    size_t ws_bytes, void *stream) {
  const hq_status s = decode_common(q, q_dtype, Hq, kv, sm_scale, n_splits, out, lse, ws, ws_bytes, Upkeep{},
                                    stream);
  if (s != HQ_OK) return s;
  return check_launch("hq_decode_attn");
}

// ---------------------------------------------------------------- allocation-free variant
// The split partials of hq_decode_attn live in a fixed device array instead
// of a caller's workspace, for callers that cannot allocate. Each device the
// library runs on holds its own copy of the array until the process ends.
// In host code the array's name is only a stand-in: its device address is
// looked up once per device with hipGetSymbolAddress (under a lock, with
// that device current) and only that address is handed to the kernels.
namespace hq {
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;       // HQ_DECODE_SCRATCH_BYTES
static_assert(kScratchBytes == HQ_DECODE_SCRATCH_BYTES, "header and library agree on the scratch size");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hq_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HQ_ERR_HIP, "hq_decode_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HQ_ERR_HIP, "hq_decode_attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HQ_OK;
}
}  // namespace
}  // namespace hq

extern "C" hq_status hq_decode_attn_noalloc(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                                            float sm_scale, int n_splits, float *out, float *lse, void *stream) {
  // every host-checkable precondition first, so that a rejected call touches no device
  const hq_status v = validate(q, q_dtype, Hq, kv, out);
  if (v != HQ_OK) return v;
  if (n_splits < 0) return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn_noalloc: n_splits < 0");
  const Plan pl = make_plan(kv, Hq, n_splits);
  if (pl.S > kMaxSplits)
    return fail(HQ_ERR_UNSUPPORTED, "hq_decode_attn_noalloc: %d splits exceed the maximum %d", pl.S, kMaxSplits);
  const size_t need = ws_layout(kv, Hq, pl).total;
  if (need > kScratchBytes)
    return fail(HQ_ERR_WORKSPACE,
                "hq_decode_attn_noalloc: these sizes need %zu bytes of split partials, above the fixed %zu "
                "(use fewer splits or hq_decode_attn with a workspace)", need, kScratchBytes);
  void *ws = nullptr;
  const hq_status s = scratch_for_current_device(&ws);
  if (s != HQ_OK) return s;
  const hq_status r = decode_common(q, q_dtype, Hq, kv, sm_scale, n_splits, out, lse, ws, kScratchBytes, Upkeep{},
                                    stream);
  if (r != HQ_OK) return r;
  return check_launch("hq_decode_attn_noalloc");
}

extern "C" hq_status hq_decode_step(const void *q, hq_dtype q_dtype, int Hq, const hq_hybrid_kv *kv,
                                    float sm_scale, int n_splits, float *out, float *lse, void *ws,
                                    size_t ws_bytes, void *q_acc, int R, int64_t step, int evict,
                                    void *stream) {
  if (q_acc && (R < 1 || R > 1024)) return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: need 1 <= R <= 1024");
  if (step < 0) return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: step < 0");
  if (q_acc && reinterpret_cast<uintptr_t>(q_acc) % 16)
    return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: q_acc must be 16-byte aligned");
  Upkeep up;
  up.q_ring = q_acc;
  up.R = q_acc ? R : 0;
  up.slot = q_acc ? static_cast<int>(step % R) : 0;
  up.evict = evict != 0 && kv && kv->W > 0;
  if (up.evict) {
    if (kv->t_cap < kv->T - kv->W + 1)
      return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: eviction needs t_cap >= T - W + 1");
    if (!kv->k_codes || !kv->v_codes || !kv->k_sz || !kv->v_sz)
      return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: null INT4 plane");
    if ((reinterpret_cast<uintptr_t>(kv->k_sz) | reinterpret_cast<uintptr_t>(kv->v_sz)) % 4)
      return fail(HQ_ERR_INVALID_ARG, "hq_decode_step: scale planes must be 4-byte aligned");
  }
  const hq_status s = decode_common(q, q_dtype, Hq, kv, sm_scale, n_splits, out, lse, ws, ws_bytes, up, stream);
  if (s != HQ_OK) return s;
  return check_launch("hq_decode_step");
}

extern "C" hq_status hq_vl_bitmap(const int32_t *vl_idx, int n_heads, int k, int64_t t_cap,
                                  uint32_t *bits, void *stream) {
  if (n_heads < 0 || k < 0 || t_cap < 0 || t_cap % 32)
    return fail(HQ_ERR_INVALID_ARG, "hq_vl_bitmap: bad sizes (t_cap must be a multiple of 32)");
  if (n_heads == 0 || t_cap == 0) { clear_error(); return HQ_OK; }
  if (!bits || (k > 0 && !vl_idx)) return fail(HQ_ERR_INVALID_ARG, "hq_vl_bitmap: null pointer");
  hipLaunchKernelGGL(vl_bitmap_kernel, dim3(n_heads), dim3(256), 0, as_stream(stream), vl_idx, k,
                     t_cap / 32, bits);
  return check_launch("hq_vl_bitmap");
}
