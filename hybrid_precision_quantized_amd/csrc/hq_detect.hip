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
//  * mfma16_colsum   (HQ_DETECT_MATMUL) bf16/fp16 MFMA 16x16x32: each wave
//    keeps the K fragments of 4 or 8 16-column tiles in registers and runs
//    over all rows of the unit (staged through LDS, 128 rows at a time) in
//    16-row chunks, accumulating every chunk into the same accumulator, so
//    the rows congruent mod 16 (rows numbered head * R + slot) are summed in
//    fp32 by the matrix core itself. The 16 residue sums of a column are then
//    added in fp64 and the total is rounded once to int64 units of 2^-16.
//    On the 2^-4 input grid, with every residue's absolute sum below 2^16,
//    each fp32 partial is exact and so is the score. colsum_resident is the
//    same arithmetic with the query rows resident in LDS for long contexts.
//  * qsum / gemv     (HQ_DETECT_QSUM) the same scores through linearity:
//    sum the unit's query rows in fp64, then one fp64 dot per key row
//    (HBM-bound: K is read once).
//  * top-k           every score kernel also writes the min and max of the
//    256 scores each of its blocks produced. topk_keys: many blocks per
//    unit reduce the unit's partial ranges, write the 32-bit keys
//    1 + (score - min) scaled by a power of two so that the range spans 31
//    bits, and a histogram of the keys' top 11 bits per block.
//    topk_select: one workgroup per unit sums the block histograms into the
//    first digit. A boundary bucket of at most 1024 keys is ranked directly
//    by (score, position), and the output offset of every block's chunk is
//    scanned; topk_write then writes each chunk's taken positions in order,
//    a workgroup per chunk. A larger bucket goes through the remaining two
//    digits (11 and 10 bits), a refinement on the bits the shift dropped and
//    a cut of equal scores by position, and its output is compacted by
//    topk_select itself, ascending by position. Up to 32768 candidates per
//    unit one launch does all of it (topk_small): each thread keeps the
//    keys of its 32 positions in registers, and the range and the first
//    histogram are built inside the workgroup.
#include "hq_common.h"

namespace hq {
namespace {

template <int DT>
__device__ __forceinline__ float load_half(uint32_t h) {
  if constexpr (DT == HQ_BF16) return bf16_to_f32(h);
  else return f16_to_f32(h);
}

// Range of the scores a 256-thread block wrote, as order-preserving
// unsigned values (score ^ sign bit): the top-k reduces these partials
// instead of reading every score once more. Every thread of the block calls.
__device__ __forceinline__ unsigned long long ordered_score(long long v) {
  return static_cast<unsigned long long>(v) ^ 0x8000000000000000ull;
}
__device__ __forceinline__ void block_range_out(unsigned long long mn, unsigned long long mx,
                                                unsigned long long *dst) {
  __shared__ unsigned long long red[8];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const unsigned long long a = __shfl_xor(mn, m, 64), c = __shfl_xor(mx, m, 64);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
  }
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = mn;
    red[2 * (threadIdx.x >> 6) + 1] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0 && dst) {
    for (int i = 1; i < static_cast<int>(blockDim.x) / 64; ++i) {
      mn = red[2 * i] < mn ? red[2 * i] : mn;
      mx = red[2 * i + 1] > mx ? red[2 * i + 1] : mx;
    }
    dst[0] = mn;
    dst[1] = mx;
  }
}

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


constexpr int kStageRows = 128;
constexpr bool kResWide8 = true;   // 512-column resident blocks as 8 waves of 4 tiles (else 4 of 8)
constexpr bool kStagedNarrow8 = true;   // 256-column staged blocks as 8 waves of 2 tiles (else 4 of 4)
constexpr int kRowPad = 8;        // halves

// Grid: units * ceil(n / (16 NT WPB)) blocks of WPB waves on the 16x16x32
// MFMA; wave w of block cb owns the NT 16-column tiles WPB NT cb + NT w + t
// with their K fragments in registers (512 columns per block while the grid
// keeps two blocks per CU, else 256; resident 512-column blocks run as 8
// waves of 4 tiles, four waves per SIMD, so that waves whose K landed early
// run their MFMAs while others still load: 20.4 -> 19.3 us at 1 x 32K, 8 KV
// heads, against 4 waves of 8 tiles, whose per-wave stamps showed each wave
// loading for ~8 us, then 5.6 us of MFMAs, then 1.5 us of epilogue, in
// lockstep across the chip; staged 256-column blocks likewise run as 8 waves
// of 2 tiles, two waves per SIMD instead of one: 20.6-21.1 -> 19.3 us at
// 1 x 32K, 2 KV heads, 1024 rows). MFMA kc covers channels 32 kc + 8 g .. + 7 for lane group g = lane
// / 16, the same order in both operands, so one K load reads 64 contiguous
// bytes of each of 16 rows (the 32x32 operand layout reads 32 bytes of each
// of 32 rows, which stalled the texture path). The unit's query rows are
// staged through LDS 128 rows at a time (double buffered; rows padded by 16
// bytes) and every A fragment feeds all NT tiles. RES (at most 256 rows):
// both slots take every row at once, the row loads are issued before the K
// loads, and both go through buffer resources that return zeros past the
// last row and the last candidate, so the loads are branch-free and each
// wait covers only what it needs (23.6 -> 20.6 us at 1 x 32K, 8 KV heads,
// against per-load branches and a wait for every K fragment before the
// first LDS store). Rows congruent mod 16 are
// summed by the matrix core itself. A lane ends with 4 of a column's 16 row
// residues; the column sums them with the other three lane groups in fp64
// (exact on the 2^-4 grid) and rounds once to int64 units of 2^-16.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int DT>
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  if constexpr (DT == HQ_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}
template <int D, int DT, int NT, bool RES, int WPB>
__global__ __launch_bounds__(64 * WPB, WPB / 2) void mfma16_colsum_kernel(const uint16_t *__restrict__ q_acc,
                                                            const uint16_t *__restrict__ k, int Hq,
                                                            int Hkv, int R, int64_t k_rows,
                                                            int64_t cand_end,
                                                            int64_t *__restrict__ scores,
                                                            unsigned long long *__restrict__ mm) {
  constexpr int KC = D / 32;                       // MFMAs per 16x16 tile and row chunk
  constexpr int NTH = 64 * WPB;                    // threads per block
  constexpr int CPB = 16 * NT * WPB;               // columns per block
  constexpr int GPB = CPB / 256;                   // 256-candidate score partials per block
  constexpr int WPG = WPB / GPB;                   // waves per partial
  static_assert(NT == 2 || NT == 4 || NT == 8, "tiles per wave");
  static_assert(WPB == 4 || WPB == 8, "waves per block");
  constexpr int ROWV = D / 8;
  constexpr int PER_T = kStageRows * ROWV / NTH;
  __shared__ uint16_t qs[2][kStageRows][D + kRowPad];
  __shared__ unsigned long long rng[WPB][2];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;                        // lane group: channels 8 g4 .. 8 g4 + 7 of each 32
  const int c16 = lane & 15;                       // column of the tile (B), row of the chunk (A)
  const int blocks_per_unit = static_cast<int>((cand_end + CPB - 1) / CPB);
  const int unit = blockIdx.x / blocks_per_unit;
  const int cb = blockIdx.x % blocks_per_unit;
  const int G = Hq / Hkv;
  const int b = unit / Hkv;
  const int h = unit % Hkv;
  const int M = G * R;
  const uint16_t *qrows = q_acc + (static_cast<int64_t>(b) * Hq + h * G) * R * D;

  uint4 buf[PER_T], buf2[PER_T];
  // RES reads through buffer resources whose ranges end at the last query
  // row and the last candidate row: the hardware returns zeros past them,
  // so the loads are straight-line code and their waits count exactly
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(qrows), static_cast<short>(0), M * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(k + static_cast<int64_t>(unit) * k_rows * D), static_cast<short>(0),
      static_cast<int>(cand_end * D * 2), 0x00020000);
  auto load_stage = [&](int st, uint4 *bb) {
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
      const int idx = e * NTH + threadIdx.x;
      const int row = idx / ROWV, c8 = idx % ROWV;
      const int grow = st * kStageRows + row;
      if constexpr (RES) {
        bb[e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              qrs, static_cast<uint32_t>((grow * D + c8 * 8) * 2), 0, 0));
      } else {
        bb[e] = grow < M ? *reinterpret_cast<const uint4 *>(qrows + static_cast<int64_t>(grow) * D + c8 * 8)
                         : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_stage = [&](int slot, const uint4 *bb) {
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
      const int idx = e * NTH + threadIdx.x;
      const int row = idx / ROWV, c8 = idx % ROWV;
      *reinterpret_cast<uint4 *>(&qs[slot][row][c8 * 8]) = bb[e];
    }
  };
  // The query rows' loads are issued before the K loads, so that storing
  // them waits for them alone (loads complete in issue order). RES: at most
  // 2 kStageRows rows, which the two slots hold at once.
  const int stages = (M + kStageRows - 1) / kStageRows;
  load_stage(0, buf);
  if constexpr (RES) load_stage(1, buf2);

  uint4 bfrag[NT][KC];
  int64_t col[NT];
  bool col_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    col[t] = static_cast<int64_t>(cb) * CPB + (wave * NT + t) * 16 + c16;
    col_ok[t] = col[t] < cand_end;
  }
  if constexpr (RES) {
    // tile by tile: the four loads of a tile read whole 256-byte rows in
    // turn (channel-block order, which lets the first MFMAs start earlier,
    // measured slower: 20.6 -> 21.5 us at 1 x 32K, 8 KV heads)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        bfrag[t][kc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     krs, static_cast<uint32_t>((col[t] * D + 32 * kc + 8 * g4) * 2),
                                                     0, 0));
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint16_t *krow = k + (static_cast<int64_t>(unit) * k_rows + (col_ok[t] ? col[t] : 0)) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        bfrag[t][kc] = col_ok[t] ? *reinterpret_cast<const uint4 *>(krow + 32 * kc + 8 * g4)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  store_stage(0, buf);
  if constexpr (RES) store_stage(1, buf2);
  __syncthreads();
  if constexpr (RES) {
    // every row is in LDS: no staging inside the loop. (Splitting the tiles
    // into parts computed in turn, so that the first part's MFMAs overlap
    // the later parts' loads, re-reads every A fragment per part and was
    // slower: 20.6 -> 21.6 us with 2 parts, 23.5 us with 4. Issuing a
    // part's K loads only once the previous part's had landed, so that the
    // first parts arrive first chip-wide, measured 20.2-20.5 us with 1, 2
    // and 4 parts alike.)
    for (int st = 0; st < stages; ++st) {
#pragma unroll
      for (int sub = 0; sub < kStageRows / 16; ++sub) {
        const uint16_t *arow = &qs[st][sub * 16 + c16][8 * g4];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint4 a = *reinterpret_cast<const uint4 *>(arow + 32 * kc);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma16<DT>(a, bfrag[t][kc], acc[t]);
        }
      }
    }
  } else {
    for (int st = 0; st < stages; ++st) {
      if (st + 1 < stages) load_stage(st + 1, buf);
      const int slot = st & 1;
#pragma unroll
      for (int sub = 0; sub < kStageRows / 16; ++sub) {
        const uint16_t *arow = &qs[slot][sub * 16 + c16][8 * g4];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint4 a = *reinterpret_cast<const uint4 *>(arow + 32 * kc);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma16<DT>(a, bfrag[t][kc], acc[t]);
        }
      }
      if (st + 1 < stages) store_stage((st + 1) & 1, buf);
      __syncthreads();
    }
  }
  // column c16 of tile t: this lane holds row residues 4 g4 .. 4 g4 + 3 (mod 16)
  unsigned long long mn = ~0ull, mx = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    double sd = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) sd += static_cast<double>(acc[t][j]);
    sd += __shfl_xor(sd, 16, 64);
    sd += __shfl_xor(sd, 32, 64);
    const long long v = __double2ll_rn(sd * 65536.0);
    if (g4 == 0 && col_ok[t]) {
      scores[static_cast<int64_t>(unit) * cand_end + col[t]] = v;
      const unsigned long long u = ordered_score(v);
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  // one partial per 256 candidates: waves WPG g .. WPG g + WPG - 1 cover group g
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const unsigned long long a = __shfl_xor(mn, m, 64), c = __shfl_xor(mx, m, 64);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
  }
  if (lane == 0) {
    rng[wave][0] = mn;
    rng[wave][1] = mx;
  }
  __syncthreads();
  const int np = static_cast<int>((cand_end + 255) / 256);   // the top-k's partial count
  const int gi = static_cast<int>(threadIdx.x);
  if (mm && gi < GPB && cb * GPB + gi < np) {
    unsigned long long a0 = rng[WPG * gi][0], c0 = rng[WPG * gi][1];
#pragma unroll
    for (int w = 1; w < WPG; ++w) {
      a0 = rng[WPG * gi + w][0] < a0 ? rng[WPG * gi + w][0] : a0;
      c0 = rng[WPG * gi + w][1] > c0 ? rng[WPG * gi + w][1] : c0;
    }
    unsigned long long *dst = mm + 2 * (static_cast<int64_t>(unit) * np + cb * GPB + gi);
    dst[0] = a0;
    dst[1] = c0;
  }
}

// ---------------------------------------------------------------- QSUM form
// Summed query rows of one unit (b, KV head): qs[d] = sum over the G * R rows
// of q_acc[b][h G + i][r][d], in fp64. One block of 256 threads per (unit,
// 8-channel slice): thread t loads the slice of rows t, t + 256, ... (one
// 16-byte load of 16-bit values, or two of fp32, per row; eight rows' loads
// in flight before their sums), the 64 lanes of a wave combine by butterfly exchanges,
// and the four waves' sums meet in LDS in wave order. Fixed order throughout
// (deterministic); exact for queries on the 2^-4 grid within the fp64 range.
template <int DT>
__global__ __launch_bounds__(256) void qsum_kernel(const void *__restrict__ q_acc, int Hq, int Hkv, int R,
                                                   int D, double *__restrict__ qs) {
  constexpr int kBatch = 8;                   // rows per thread in flight
  __shared__ double part[4][8];
  const int slices = D / 8;
  const int unit = blockIdx.x / slices;
  const int sl = blockIdx.x % slices;
  const int G = Hq / Hkv;
  const int b = unit / Hkv;
  const int h = unit % Hkv;
  const int M = G * R;
  const int t = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * Hq + h * G) * R * D + sl * 8;
  double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int r0 = t; r0 < M; r0 += 256 * kBatch) {
    if constexpr (DT == HQ_F32) {
      float4 x[kBatch][2];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int r = r0 + 256 * j;
        if (r < M) {
          const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(q_acc) + base +
                                                             static_cast<int64_t>(r) * D);
          x[j][0] = p[0];
          x[j][1] = p[1];
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (r0 + 256 * j < M) {
          const float v[8] = {x[j][0].x, x[j][0].y, x[j][0].z, x[j][0].w,
                              x[j][1].x, x[j][1].y, x[j][1].z, x[j][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] += static_cast<double>(v[e]);
        }
      }
    } else {
      uint4 u[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int r = r0 + 256 * j;
        if (r < M)
          u[j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q_acc) + base +
                                                  static_cast<int64_t>(r) * D);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (r0 + 256 * j < M) {
          const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[2 * e] += static_cast<double>(load_half<DT>(w[e] & 0xFFFFu));
            s[2 * e + 1] += static_cast<double>(load_half<DT>(w[e] >> 16));
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += __shfl_xor(s[e], m, 64);
  if ((t & 63) == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) part[t >> 6][e] = s[e];
  __syncthreads();
  if (t < 8) qs[static_cast<int64_t>(unit) * D + sl * 8 + t] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
}

// 256 threads; lanes in groups of D/8 per key row (8 channels per lane).
// The same column sums with the unit's query rows resident: all M <= 256
// rows are staged into LDS once, then the block walks `gpb` groups of 256
// columns (16 tiles of 16, four per wave, on the 16x16x32 MFMA with the
// channel order of mfma16_colsum), loading the next group's K
// fragments into a second register set while the matrix core works on the
// current one. Q is read from L2 once per gpb groups instead of once per
// group, and the K stream overlaps the MFMAs. Each group writes its scores;
// its score range (one partial per 256 candidates, as the top-k expects)
// goes per wave into LDS and is reduced over the waves after the last group,
// so the waves of a block meet at no barrier between groups.
constexpr int kResRows = 256;
constexpr int kResMaxGroups = 16;                 // groups per block at most
template <int D, int DT>
__global__ __launch_bounds__(256, 2) void colsum_resident_kernel(const uint16_t *__restrict__ q_acc,
                                                                 const uint16_t *__restrict__ k, int Hq,
                                                                 int Hkv, int R, int64_t k_rows,
                                                                 int64_t cand_end, int groups, int gpb,
                                                                 int64_t *__restrict__ scores,
                                                                 unsigned long long *__restrict__ mm) {
  constexpr int KC = D / 32;                       // 16x16x32 MFMAs per tile and row chunk
  constexpr int NT = 4;                            // 16-column tiles per wave and group
  constexpr int ROWV = D / 8;
  __shared__ uint16_t qs[kResRows][D + kRowPad];
  __shared__ unsigned long long rng[kResMaxGroups][4][2];     // [group in block][wave] {min, max}
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;                        // lane group: channels 8 g4 .. + 7 of each 32
  const int c16 = lane & 15;                       // column of a tile (B), row of a chunk (A)
  const int bpu = (groups + gpb - 1) / gpb;                   // blocks per unit
  const int unit = blockIdx.x / bpu;
  const int g0 = (blockIdx.x % bpu) * gpb;
  const int g1 = g0 + gpb < groups ? g0 + gpb : groups;
  const int G = Hq / Hkv;
  const int b = unit / Hkv;
  const int h = unit % Hkv;
  const int M = G * R;                                        // <= kResRows
  const int subs = (M + 15) / 16;
  const uint16_t *qrows = q_acc + (static_cast<int64_t>(b) * Hq + h * G) * R * D;
  // The K fragments are read and the scores written through buffer
  // resources that end at the unit's last candidate: past it, loads return
  // zeros and stores are dropped, and the loads and stores are branch-free
  // (qwen-sized 16 x 128K column sums 1033 -> 1006 us against per-load
  // branches). The compiler still places waits that cover part of the next
  // group's prefetch before a group's MFMAs.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(k + static_cast<int64_t>(unit) * k_rows * D), static_cast<short>(0),
      static_cast<int>(cand_end * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      scores + static_cast<int64_t>(unit) * cand_end, static_cast<short>(0), static_cast<int>(cand_end * 8),
      0x00020000);

  // K fragments of group g: this lane's column of tiles 4 wave + t of the
  // group, channels 32 kc + 8 g4 .. + 7 (64 contiguous bytes per row and kc)
  auto load_frag = [&](int g, uint4 (&kf)[NT][KC]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t col = static_cast<uint32_t>(g * 256 + (wave * NT + t) * 16 + c16);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[t][kc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  krs, (col * D + 32 * kc + 8 * g4) * 2, 0, 0));
    }
  };
  uint4 kfa[NT][KC], kfb[NT][KC];
  if (g0 < g1) load_frag(g0, kfa);
  // all query rows into LDS (zero past M)
  for (int idx = threadIdx.x; idx < kResRows * ROWV; idx += 256) {
    const int row = idx / ROWV, c8 = idx % ROWV;
    *reinterpret_cast<uint4 *>(&qs[row][c8 * 8]) =
        row < M ? *reinterpret_cast<const uint4 *>(qrows + static_cast<int64_t>(row) * D + c8 * 8)
                : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  auto group = [&](int g, const uint4 (&kf)[NT][KC], uint4 (&next)[NT][KC]) {
    if (g + 1 < g1) load_frag(g + 1, next);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sub = 0; sub < subs; ++sub) {
      const uint16_t *arow = &qs[sub * 16 + c16][8 * g4];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 a = *reinterpret_cast<const uint4 *>(arow + 32 * kc);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma16<DT>(a, kf[t][kc], acc[t]);
      }
    }
    // column c16 of tile t: this lane holds row residues 4 g4 .. 4 g4 + 3 (mod 16)
    unsigned long long mn = ~0ull, mx = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t col = static_cast<int64_t>(g) * 256 + (wave * NT + t) * 16 + c16;
      double sd = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) sd += static_cast<double>(acc[t][j]);
      sd += __shfl_xor(sd, 16, 64);
      sd += __shfl_xor(sd, 32, 64);
      const long long v = __double2ll_rn(sd * 65536.0);
      // lane group 0 stores; the others aim past the range (dropped)
      const uint32_t so = g4 == 0 ? static_cast<uint32_t>(col) * 8u : 0x80000000u;
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), srs, so, 0, 0);
      const bool ok = col < cand_end;
      const unsigned long long u = ordered_score(v);
      mn = ok && u < mn ? u : mn;
      mx = ok && u > mx ? u : mx;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const unsigned long long a = __shfl_xor(mn, m, 64), c = __shfl_xor(mx, m, 64);
      mn = a < mn ? a : mn;
      mx = c > mx ? c : mx;
    }
    if (lane == 0) {
      rng[g - g0][wave][0] = mn;
      rng[g - g0][wave][1] = mx;
    }
  };
  for (int g = g0; g < g1; g += 2) {
    group(g, kfa, kfb);
    if (g + 1 < g1) group(g + 1, kfb, kfa);
  }
  __syncthreads();
  const int gi = static_cast<int>(threadIdx.x);
  if (mm && gi < g1 - g0) {
    unsigned long long mn = rng[gi][0][0], mx = rng[gi][0][1];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      mn = rng[gi][w][0] < mn ? rng[gi][w][0] : mn;
      mx = rng[gi][w][1] > mx ? rng[gi][w][1] : mx;
    }
    unsigned long long *dst = mm + 2 * (static_cast<int64_t>(unit) * groups + g0 + gi);
    dst[0] = mn;
    dst[1] = mx;
  }
}

template <int D, int DT>
__global__ __launch_bounds__(256) void gemv_kernel(const void *__restrict__ k, const double *__restrict__ qs,
                                                   int64_t k_rows, int64_t cand_end, int chunks_per_unit,
                                                   int64_t *__restrict__ scores,
                                                   unsigned long long *__restrict__ mm) {
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
  unsigned long long mn = ~0ull, mx = 0;
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
    if (ok && sub == 0) {
      const long long v = __double2ll_rn(acc * 65536.0);
      scores[static_cast<int64_t>(unit) * cand_end + r] = v;
      const unsigned long long u = ordered_score(v);
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  block_range_out(mn, mx, mm ? mm + 2 * static_cast<int64_t>(blockIdx.x) : nullptr);
}

// ---------------------------------------------------------------- top-k
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
constexpr int kTopkThreads = 1024;
constexpr int kRun = 32;                       // positions per thread per batch
constexpr int kDigitBits = 11;                 // three passes over a 32-bit key
constexpr int kBins = 1 << kDigitBits;
constexpr int kHists = kTopkThreads / 128;     // one histogram per two waves
// per-unit stride of the streamed keys (a multiple of 4: 16-byte loads)
__host__ __device__ inline int64_t key_stride(int64_t n) { return (n + 3) & ~3LL; }

// exclusive scan of one int per thread over the block; *total gets the sum
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
  if (threadIdx.x < 64) {                       // scan of the 16 wave totals by the first wave
    const int t = threadIdx.x < kTopkThreads / 64 ? sh[threadIdx.x] : 0;
    int x = t;
#pragma unroll
    for (int m = 1; m < kTopkThreads / 64; m <<= 1) {
      const int y = __shfl_up(x, m, 64);
      if (static_cast<int>(threadIdx.x) >= m) x += y;
    }
    if (threadIdx.x < kTopkThreads / 64) sh[threadIdx.x] = x - t;
    if (threadIdx.x == kTopkThreads / 64 - 1) sh[kTopkThreads / 64] = x;
  }
  __syncthreads();
  const int pre = sh[w] + inc - v;
  *total = sh[kTopkThreads / 64];
  __syncthreads();
  return pre;
}

constexpr int kSmallBucket = kTopkThreads;     // boundary buckets up to this size are ranked directly
struct TopkShared {
  uint32_t whist[kHists][kBins];
  uint32_t hist[kBins];
  int scan[kTopkThreads / 64 + 2];
  int sel[4];
  unsigned long long mm[2 * kTopkThreads / 64];
  long long bsc[kSmallBucket];                 // the boundary bucket: scores and positions
  int bpos[kSmallBucket];
  int rank[kSmallBucket];
  int cnt[32];                                 // taken positions per chunk (the write launch's offsets)
  int bcnt;
};

template <class SH>
__device__ __forceinline__ void clear_whist(SH &sh) {
  uint32_t *h = &sh.whist[0][0];
  for (int i = threadIdx.x; i < kHists * kBins; i += kTopkThreads) h[i] = 0u;
}
// sum the histograms into sh.hist
template <class SH>
__device__ __forceinline__ void reduce_whist(SH &sh) {
  for (int b = threadIdx.x; b < kBins; b += kTopkThreads) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kHists; ++w) t += sh.whist[w][b];
    sh.hist[b] = t;
  }
}
// Digit search after a histogram pass: the digit (bins in descending order)
// holding the k_rem-th largest; returns it, *k_rem becomes the rank inside
// the digit and *cnt the digit's population. The first wave searches (lane
// l holds the l-th group of bins from the top) and publishes the result
// behind one barrier; sel is written again only behind later barriers.
template <class SH>
__device__ int find_digit(int nb, int *k_rem, int *cnt, SH &sh) {
  constexpr int kPer = kBins / 64;                 // bins per lane at most
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (nb + 63) / 64;
    const int hi = nb - per * lane > 0 ? nb - per * lane : 0;          // bins [lo, hi)
    const int lo = hi - per > 0 ? hi - per : 0;
    const int nv = hi - lo;
    uint32_t v[kPer];                              // every read issued at once
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = i < nv ? sh.hist[lo + i] : 0u;
    int s = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) s += static_cast<int>(v[i]);
    int inc = s;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int y = __shfl_up(inc, m, 64);
      if (lane >= m) inc += y;
    }
    const int kr = *k_rem;
    int acc = inc - s;                                                  // above this lane's bins
    if (acc < kr && kr <= inc) {                   // one lane: walk its bins from the top
      int bsel = 0, rsel = 0, csel = 0;
#pragma unroll
      for (int i = kPer - 1; i >= 0; --i) {
        const int c = static_cast<int>(v[i]);
        if (acc < kr && kr <= acc + c) {
          bsel = lo + i;
          rsel = kr - acc;
          csel = c;
        }
        acc += c;
      }
      sh.sel[0] = bsel;
      sh.sel[1] = rsel;
      sh.sel[2] = csel;
    }
  }
  __syncthreads();
  *k_rem = sh.sel[1];
  *cnt = sh.sel[2];
  return sh.sel[0];
}

// Chunking of a unit's candidates over the blocks of the keys and write launches.
constexpr int kTkBlock = 256;
constexpr int kTkMaxBlocks = 32;
static_assert(kTkMaxBlocks <= 32, "TopkShared::cnt and the select kernel's per-chunk sums hold 32 chunks");
struct TopkChunks {
  int nbu;        // blocks per unit
  int64_t ch;     // candidates per block (a multiple of 4)
};
__host__ __device__ inline TopkChunks topk_chunks(int64_t n) {
  int64_t nbu = (n + 1023) / 1024;
  if (nbu > kTkMaxBlocks) nbu = kTkMaxBlocks;
  if (nbu < 1) nbu = 1;
  TopkChunks c;
  c.nbu = static_cast<int>(nbu);
  c.ch = (((n + nbu - 1) / nbu) + 3) & ~3LL;
  return c;
}
// Partial score ranges per unit: one per 256 candidates, written by the
// score kernels (every one of them covers 256 candidates per block).
__host__ __device__ inline int topk_partials(int64_t n) { return static_cast<int>((n + 255) / 256); }
// Per unit, what the select launch hands the write launch: {mode, first
// digit, output offset of every chunk}; mode 0: the write launch writes the
// chunk's taken positions, 1: the select launch has written them.
constexpr int kCtl = kTkMaxBlocks + 2;
// workspace of the top-k: partial ranges, block histograms, keys, control
struct TopkWs {
  size_t mm, hist, keys, ctl, total;
};
TopkWs topk_ws(int64_t units, int64_t n) {
  const TopkChunks c = topk_chunks(n);
  TopkWs L{};
  L.mm = 0;
  L.hist = align_up(static_cast<size_t>(units) * topk_partials(n) * 2 * sizeof(unsigned long long), 256);
  L.keys = align_up(L.hist + static_cast<size_t>(units) * c.nbu * kBins * sizeof(uint32_t), 256);
  L.ctl = align_up(L.keys + static_cast<size_t>(units) * key_stride(n) * sizeof(uint32_t), 256);
  L.total = align_up(L.ctl + static_cast<size_t>(units) * kCtl * sizeof(int), 256);
  return L;
}
// where the score kernels put their partial ranges
unsigned long long *topk_mm(void *tws, int64_t units, int64_t n) {
  return reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(tws) + topk_ws(units, n).mm);
}

__device__ __forceinline__ unsigned long long ordered(long long v) {
  return static_cast<unsigned long long>(v) ^ 0x8000000000000000ull;
}
// The unit's key parameters from its score range [mn, mx]: keys 1 + (((score
// - mn) >> shift) << lsh), so the range spans bits 0..30 whatever its width
// (a wider one drops its low bits, a narrower one is moved up so that the
// first digit splits it as finely as a wide one), the largest key is at most
// 2^31, and key 0 marks no position.
__device__ __forceinline__ void key_params(unsigned long long mn, unsigned long long mx, int &shift, int &lsh) {
  const unsigned long long range = mx - mn;
  const int nbits = range == 0 ? 0 : 64 - __clzll(static_cast<long long>(range));
  shift = nbits > 31 ? nbits - 31 : 0;
  lsh = nbits < 31 ? 31 - nbits : 0;
}
// Min and max over the nbu partial ranges {mn, mx} at mm, by one wave: the
// partials come through a buffer resource in batches of kRangeBatch per
// lane, every load of a batch in flight at once (a loop with a load and a
// use per step waits for every load issued before it, the caller's too).
// Every lane ends with the result; the reduction order is fixed.
constexpr int kRangeBatch = 8;
__device__ __forceinline__ void wave_range(const unsigned long long *mm, int nbu, unsigned long long &mn,
                                           unsigned long long &mx) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned long long *>(mm), static_cast<short>(0), nbu * 16, 0x00020000);
  mn = ~0ull;
  mx = 0;
  for (int i0 = 0; i0 < nbu; i0 += 64 * kRangeBatch) {
    uint4 v[kRangeBatch];
#pragma unroll
    for (int e = 0; e < kRangeBatch; ++e)
      v[e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, static_cast<uint32_t>(i0 + e * 64 + lane) * 16u, 0, 0));
#pragma unroll
    for (int e = 0; e < kRangeBatch; ++e) {
      const bool ok = i0 + e * 64 + lane < nbu;
      const unsigned long long a = ok ? (static_cast<unsigned long long>(v[e].y) << 32 | v[e].x) : ~0ull;
      const unsigned long long c = ok ? (static_cast<unsigned long long>(v[e].w) << 32 | v[e].z) : 0ull;
      mn = a < mn ? a : mn;
      mx = c > mx ? c : mx;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const unsigned long long a = __shfl_xor(mn, m, 64), c = __shfl_xor(mx, m, 64);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
  }
}
// the unit's range from its nbu partials, by the first wave (every block
// and every launch reduces them in the same way)
__device__ __forceinline__ void unit_range(const unsigned long long *mm, int nbu, unsigned long long &base,
                                           int &shift, int &lsh, unsigned long long *red) {
  if (threadIdx.x < 64) {
    unsigned long long mn, mx;
    wave_range(mm, nbu, mn, mx);
    if (threadIdx.x == 0) {
      red[0] = mn;
      red[1] = mx;
    }
  }
  __syncthreads();
  base = red[0];
  key_params(red[0], red[1], shift, lsh);
  __syncthreads();
}
__device__ __forceinline__ uint32_t score_key(unsigned long long off, int shift, int lsh) {
  return 1u + (static_cast<uint32_t>(off >> shift) << lsh);
}

// 1. per (unit, block): the chunk's keys and the histogram of their top 11 bits
__global__ __launch_bounds__(kTkBlock) void topk_keys_kernel(const int64_t *__restrict__ scores, int64_t n,
                                                             int nbu, int64_t ch, int np,
                                                             const unsigned long long *__restrict__ mm,
                                                             uint32_t *__restrict__ keys,
                                                             uint32_t *__restrict__ bhist) {
  __shared__ uint32_t h[kTkBlock / 64][kBins];
  __shared__ unsigned long long red[2];
  const int unit = blockIdx.x / nbu, blk = blockIdx.x % nbu;
  const int64_t *sc = scores + static_cast<int64_t>(unit) * n;
  uint32_t *kk = keys + static_cast<int64_t>(unit) * key_stride(n);
  for (int i = threadIdx.x; i < (kTkBlock / 64) * kBins; i += kTkBlock) (&h[0][0])[i] = 0u;
  const int64_t c0 = blk * ch;
  const int64_t c1 = c0 + ch < n ? c0 + ch : n;
  const int cn = static_cast<int>(c1 > c0 ? c1 - c0 : 0);           // this chunk's candidates
  // The chunk's scores come through a buffer resource, kKeysBatch per
  // thread in flight at once (loads past the chunk return 0 and are not
  // used); the first batch flies while the range is reduced. (One guarded
  // load per step waited for each load in turn.)
  constexpr int kKeysBatch = 8;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int64_t *>(sc + c0), static_cast<short>(0), cn * 8, 0x00020000);
  unsigned long long v[kKeysBatch];
  auto load_batch = [&](int q0) {
#pragma unroll
    for (int e = 0; e < kKeysBatch; ++e)
      v[e] = __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(
                                    rs, static_cast<uint32_t>(q0 + e * kTkBlock + threadIdx.x) * 8u, 0, 0));
  };
  load_batch(0);
  unsigned long long base;
  int shift, lsh;
  unit_range(mm + 2 * static_cast<int64_t>(unit) * np, np, base, shift, lsh, red);
  uint32_t *wh = h[threadIdx.x >> 6];
  for (int q0 = 0; q0 < cn; q0 += kKeysBatch * kTkBlock) {         // same trip count in every thread
#pragma unroll
    for (int e = 0; e < kKeysBatch; ++e) {
      const int q = q0 + e * kTkBlock + static_cast<int>(threadIdx.x);
      const uint32_t key = score_key(ordered(static_cast<long long>(v[e])) - base, shift, lsh);
      if (q < cn) {
        kk[c0 + q] = key;
        atomicAdd(&wh[key >> 21], 1u);
      }
    }
    load_batch(q0 + kKeysBatch * kTkBlock);
  }
  __syncthreads();
  uint32_t *bh = bhist + (static_cast<int64_t>(unit) * nbu + blk) * kBins;
  for (int b = threadIdx.x; b < kBins; b += kTkBlock) bh[b] = h[0][b] + h[1][b] + h[2][b] + h[3][b];
}

// Visits the thread's positions [t P, t P + P) of a unit's keys, streamed
// from the workspace in batches of kRun with 16-byte loads: visit(j, key,
// valid). The trip count is the same for every thread (P is uniform), so the
// body may use wave-wide operations.
template <class F>
__device__ __forceinline__ void for_own_ws(const uint32_t *gk, int64_t nst, int64_t P, int64_t j1, F &&visit) {
#pragma unroll 1
  for (int64_t c0 = 0; c0 < P; c0 += kRun) {
    const int64_t b0 = threadIdx.x * P + c0;          // a multiple of 4
    uint32_t kv[kRun];
#pragma unroll
    for (int i = 0; i < kRun / 4; ++i) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (b0 + 4 * i < nst) v = *reinterpret_cast<const uint4 *>(gk + b0 + 4 * i);
      kv[4 * i] = v.x; kv[4 * i + 1] = v.y; kv[4 * i + 2] = v.z; kv[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < kRun; ++i) visit(b0 + i, kv[i], b0 + i < j1);
  }
}

// Visits every position j < n of a unit's keys in the workspace, in no
// particular order: 16-byte loads, consecutive across the block (coalesced),
// kBatch of them in flight per thread: visit(j, key).
template <class F>
__device__ __forceinline__ void for_all_ws(const uint32_t *gk, int64_t n, F &&visit) {
  constexpr int kBatch = 8;
  const uint4 *g4 = reinterpret_cast<const uint4 *>(gk);
  const int64_t n4 = key_stride(n) / 4;
#pragma unroll 1
  for (int64_t i0 = 0; i0 < n4; i0 += static_cast<int64_t>(kBatch) * kTopkThreads) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * kTopkThreads + threadIdx.x;
      v[u] = i < n4 ? g4[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = 4 * (i0 + static_cast<int64_t>(u) * kTopkThreads + threadIdx.x);
      const uint32_t kk[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j + c < n) visit(j + c, kk[c]);
    }
  }
}

// The radix path after the first digit (prefix = that digit << 21): the
// other two digits (bits 10..20, then 0..9) over the streamed keys; then,
// when the threshold key's bucket is not taken whole, a selection on the low
// `shift` bits of the scores that the keys dropped; then the in-order
// compaction: every candidate above the threshold, and of those equal to it
// the first `take` by position.
// The histogram passes stream the keys coalesced (for_all_ws) with one LDS
// atomic per key; the counts and the compaction walk each thread's own
// positions in order (for_own_ws).
__device__ void topk_radix(TopkShared &sh, const int64_t *sc, const uint32_t *gk, int64_t n, int64_t nst,
                           int64_t P, int64_t j1, unsigned long long base, int shift, uint32_t prefix, int k_rem,
                           int eq, int k_top, int32_t *out) {
  uint32_t *wh = sh.whist[threadIdx.x >> 7];
  uint32_t pmask = 0x7FFu << 21;
  auto off = [&](long long sv) -> unsigned long long { return ordered(sv) - base; };
  auto for_own = [&](auto &&visit) { for_own_ws(gk, nst, P, j1, visit); };
#pragma unroll 1
  for (int ps = 0; ps < 2; ++ps) {
    const int sft = ps == 0 ? 10 : 0;
    const int nbt = ps == 0 ? 11 : 10;
    const uint32_t dm = (1u << nbt) - 1u;
    clear_whist(sh);
    __syncthreads();
    for_all_ws(gk, n, [&](int64_t, uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&wh[(key >> sft) & dm], 1u);
    });
    __syncthreads();
    reduce_whist(sh);
    __syncthreads();
    const int d = find_digit(1 << nbt, &k_rem, &eq, sh);
    prefix |= static_cast<uint32_t>(d) << sft;
    pmask |= dm << sft;
  }
  const uint32_t kappa = prefix;   // key of the k_top-th largest (>= 1)
  int take = k_rem;                // taken among key == kappa
  // members of the kappa bucket differ only in the low `shift` bits: select
  // on those bits when the bucket is not taken whole
  const bool refine = eq > take && shift > 0;
  unsigned long long low = 0;
  if (refine) {
    unsigned long long lowpre = 0, lowmask = 0;
    const unsigned long long lbits = (shift >= 64) ? ~0ull : ((1ull << shift) - 1ull);
    for (int top = shift; top > 0; top -= kDigitBits) {
      const int bits = top >= kDigitBits ? kDigitBits : top;
      const int sh2 = top - bits;
      clear_whist(sh);
      __syncthreads();
      for_all_ws(gk, n, [&](int64_t j, uint32_t key) {
        if (key == kappa) {
          const unsigned long long lo = off(sc[j]) & lbits;
          if ((lo & lowmask) == lowpre) atomicAdd(&wh[static_cast<uint32_t>(lo >> sh2) & ((1u << bits) - 1u)], 1u);
        }
      });
      __syncthreads();
      reduce_whist(sh);
      __syncthreads();
      int cnt;
      const int d = find_digit(1 << bits, &take, &cnt, sh);
      lowpre |= static_cast<unsigned long long>(d) << sh2;
      lowmask |= static_cast<unsigned long long>((1u << bits) - 1u) << sh2;
    }
    low = lowpre;
  }
  const unsigned long long tau = (static_cast<unsigned long long>(kappa - 1u) << shift) + low;
  auto is_tie = [&](int64_t j, uint32_t key) -> bool {
    if (key != kappa) return false;
    return refine ? (off(sc[j]) == tau) : true;
  };
  auto is_sure = [&](int64_t j, uint32_t key) -> bool {
    if (key != kappa) return key > kappa;
    return refine && off(sc[j]) > tau;
  };
  int ties = 0, sure = 0;
  for_own([&](int64_t j, uint32_t key, bool ok) {
    if (ok) {
      ties += is_tie(j, key);
      sure += is_sure(j, key);
    }
  });
  int tot;
  const int tie_before = block_exclusive_scan(ties, sh.scan, &tot);
  int sel = sure;
  {
    int r = tie_before;
    for_own([&](int64_t j, uint32_t key, bool ok) {
      if (ok && is_tie(j, key)) { sel += (r < take); ++r; }
    });
  }
  int pos = block_exclusive_scan(sel, sh.scan, &tot);
  {
    int r = tie_before;
    for_own([&](int64_t j, uint32_t key, bool ok) {
      if (!ok) return;
      bool sj = is_sure(j, key);
      if (is_tie(j, key)) { sj = r < take; ++r; }
      if (sj && pos < k_top) out[pos++] = static_cast<int32_t>(j);
    });
  }
}

// Ranks the boundary bucket's eq members (sh.bsc, sh.bpos; sh.rank zeroed)
// in the order (score descending, position ascending): parts = 1024 / eq
// threads share a member's comparisons. Ends behind a barrier.
__device__ __forceinline__ void rank_bucket(TopkShared &sh, int eq) {
  const int parts = kTopkThreads / eq;
  const int e = static_cast<int>(threadIdx.x) / parts;
  const int part = static_cast<int>(threadIdx.x) % parts;
  if (e < eq) {
    const long long ms = sh.bsc[e];
    const int mp = sh.bpos[e];
    int r = 0;
    for (int i = part; i < eq; i += parts) {
      const long long si = sh.bsc[i];
      r += (si > ms) || (si == ms && sh.bpos[i] < mp);
    }
    if (r) atomicAdd(&sh.rank[e], r);
  }
  __syncthreads();
}

// 2. One workgroup per unit. The first digit comes from the block
// histograms (every load in flight at once). When its bucket holds at most
// kSmallBucket keys, the bucket's (score, position) pairs are collected (a
// coalesced pass over the keys, any order) and ranked, each member's
// decision is written into its key (all ones: taken, 0: dropped), and the
// number of taken positions of every chunk of the keys launch (its keys
// above the digit, from its histogram, plus its taken members) is scanned
// into the chunks' output offsets: the write launch then emits the positions
// in order, a workgroup per chunk. A larger bucket takes the radix path here,
// which writes the output itself.
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(const int64_t *__restrict__ scores,
                                                                   uint32_t *__restrict__ keys,
                                                                   const uint32_t *__restrict__ bhist,
                                                                   const unsigned long long *__restrict__ mm,
                                                                   int64_t n, int nbu, int64_t ch, int np,
                                                                   int k_top, int32_t *__restrict__ idx_out,
                                                                   int *__restrict__ ctl) {
  __shared__ TopkShared sh;
  const int unit = blockIdx.x;
  const int64_t *sc = scores + static_cast<int64_t>(unit) * n;
  const int64_t nst = key_stride(n);
  uint32_t *gk = keys + static_cast<int64_t>(unit) * nst;
  int32_t *out = idx_out + static_cast<int64_t>(unit) * k_top;
  int *cu = ctl + static_cast<int64_t>(unit) * kCtl;
  if (k_top == 0) return;
  const uint32_t *bh = bhist + static_cast<int64_t>(unit) * nbu * kBins;
  for (int b = threadIdx.x; b < kBins; b += kTopkThreads) {
    uint32_t v[kTkMaxBlocks];
#pragma unroll
    for (int blk = 0; blk < kTkMaxBlocks; ++blk) v[blk] = blk < nbu ? bh[static_cast<int64_t>(blk) * kBins + b] : 0u;
    uint32_t t = 0;
#pragma unroll
    for (int blk = 0; blk < kTkMaxBlocks; ++blk) t += v[blk];
    sh.hist[b] = t;
  }
  if (threadIdx.x == 0) sh.bcnt = 0;
  if (threadIdx.x < kSmallBucket) sh.rank[threadIdx.x] = 0;
  if (threadIdx.x < kTkMaxBlocks) sh.cnt[threadIdx.x] = 0;
  __syncthreads();
  int k_rem = k_top, eq = 0;
  const uint32_t d1 = static_cast<uint32_t>(find_digit(kBins, &k_rem, &eq, sh));

  if (eq <= kSmallBucket) {                     // eq: from LDS, uniform
    constexpr int kBatch = 8;                   // 16-byte key loads in flight per thread
    const uint4 *g4 = reinterpret_cast<const uint4 *>(gk);
    const int64_t n4 = nst / 4;
#pragma unroll 1
    for (int64_t i0 = 0; i0 < n4; i0 += static_cast<int64_t>(kBatch) * kTopkThreads) {
      uint4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * kTopkThreads + threadIdx.x;
        v[u] = i < n4 ? g4[i] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t j = 4 * (i0 + static_cast<int64_t>(u) * kTopkThreads + threadIdx.x);
        const uint32_t kk[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (j + c < n && (kk[c] >> 21) == d1) {
            const int slot = atomicAdd(&sh.bcnt, 1);
            sh.bsc[slot] = sc[j + c];
            sh.bpos[slot] = static_cast<int>(j + c);
          }
        }
      }
    }
    __syncthreads();
    rank_bucket(sh, eq);
    // per chunk: its keys above the digit (32 threads sum a chunk's bins
    // above d1), then its taken members
    {
      const int blk = static_cast<int>(threadIdx.x) >> 5, part = threadIdx.x & 31;
      uint32_t a = 0;
      if (blk < nbu) {
        const uint32_t *h = bh + static_cast<int64_t>(blk) * kBins;
#pragma unroll 8
        for (int b = static_cast<int>(d1) + 1 + part; b < kBins; b += 32) a += h[b];
      }
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) a += __shfl_xor(a, m, 64);
      if (part == 0 && blk < nbu) atomicAdd(&sh.cnt[blk], static_cast<int>(a));
    }
    if (static_cast<int>(threadIdx.x) < eq) {
      const bool t = sh.rank[threadIdx.x] < k_rem;
      gk[sh.bpos[threadIdx.x]] = t ? 0xFFFFFFFFu : 0u;
      if (t) atomicAdd(&sh.cnt[static_cast<int64_t>(sh.bpos[threadIdx.x]) / ch], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int c = static_cast<int>(threadIdx.x) < nbu ? sh.cnt[threadIdx.x] : 0;
      int inc = c;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int y = __shfl_up(inc, m, 64);
        if (static_cast<int>(threadIdx.x) >= m) inc += y;
      }
      if (threadIdx.x == 0) {
        cu[0] = 0;
        cu[1] = static_cast<int>(d1);
      }
      if (static_cast<int>(threadIdx.x) < nbu) cu[2 + threadIdx.x] = inc - c;
    }
    return;
  }
  if (threadIdx.x == 0) cu[0] = 1;
  const int64_t P = ((n + kTopkThreads - 1) / kTopkThreads + 3) & ~3LL;   // wave-uniform
  const int64_t j0 = threadIdx.x * P < n ? threadIdx.x * P : n;
  const int64_t j1 = j0 + P < n ? j0 + P : n;
  unsigned long long base;
  int shift, lsh;
  unit_range(mm + 2 * static_cast<int64_t>(unit) * np, np, base, shift, lsh, sh.mm);
  topk_radix(sh, sc, gk, n, nst, P, j1, base, shift, d1 << 21, k_rem, eq, k_top, out);
}

// 3. Per (unit, chunk of the keys launch), when the select launch left the
// writing to it: thread t tests positions [c0 + t Q, c0 + t Q + Q) (taken:
// key all ones, or first digit above d1), the block scans the counts, and
// the taken positions go to out[offset + rank] in ascending order.
constexpr int kWrThreads = 256;
constexpr int kWrRun = 16;                     // positions per thread per batch
__global__ __launch_bounds__(kWrThreads) void topk_write_kernel(const uint32_t *__restrict__ keys,
                                                                const int *__restrict__ ctl, int64_t n, int nbu,
                                                                int64_t ch, int k_top,
                                                                int32_t *__restrict__ idx_out) {
  __shared__ int scan[kWrThreads / 64 + 1];
  const int unit = blockIdx.x / nbu, blk = blockIdx.x % nbu;
  const int *cu = ctl + static_cast<int64_t>(unit) * kCtl;
  if (k_top == 0) return;
  const uint32_t *gk = keys + static_cast<int64_t>(unit) * key_stride(n);
  int32_t *out = idx_out + static_cast<int64_t>(unit) * k_top;
  const int64_t c0 = static_cast<int64_t>(blk) * ch;
  const int64_t c1 = c0 + ch < n ? c0 + ch : n;
  const int64_t Q = ((ch + kWrThreads - 1) / kWrThreads + 3) & ~3LL;       // a multiple of 4
  const int64_t b0 = c0 + static_cast<int64_t>(threadIdx.x) * Q;
  // taken bits of positions [b0 + q0, b0 + q0 + kWrRun): the chunk's keys
  // come through a buffer resource over whole 16-byte groups (c0 is a
  // multiple of 4 and the unit's key stride too, so the groups stay inside
  // it); loads past it return 0 and keys past c1 are masked, so the loads
  // are branch-free and all in flight at once
  const int cn = static_cast<int>(c1 > c0 ? c1 - c0 : 0);
  const __amdgpu_buffer_rsrc_t ks = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(gk + c0), static_cast<short>(0), ((cn + 3) & ~3) * 4, 0x00020000);
  const uint32_t t0 = static_cast<uint32_t>(threadIdx.x) * static_cast<uint32_t>(Q);
  auto load_run = [&](int64_t q0, uint4 *v) {
#pragma unroll
    for (int i = 0; i < kWrRun / 4; ++i)
      v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           ks, (t0 + static_cast<uint32_t>(q0) + 4u * i) * 4u, 0, 0));
  };
  auto run_bits = [&](int64_t q0, const uint4 *v, uint32_t d1) -> uint32_t {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kWrRun / 4; ++i) {
      const uint32_t kk[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t q = q0 + 4 * i + c;
        const bool t = q < Q && t0 + q < cn && (kk[c] == 0xFFFFFFFFu || (kk[c] >> 21) > d1);
        m |= static_cast<uint32_t>(t) << (4 * i + c);
      }
    }
    return m;
  };
  auto taken = [&](int64_t q0, uint32_t d1) -> uint32_t {
    uint4 v[kWrRun / 4];
    load_run(q0, v);
    return run_bits(q0, v, d1);
  };
  // the first run's keys are in flight while the select launch's control
  // words are read (no early return, which the compiler would hoist above
  // the loads; a block whose unit the select launch wrote itself writes
  // nothing), and its bits stay in a register for the write pass (at most
  // one run per thread unless a chunk exceeds kWrThreads kWrRun keys)
  uint4 v0[kWrRun / 4];
  load_run(0, v0);
  const bool mine = cu[0] == 0;                // uniform over the block
  const uint32_t d1 = static_cast<uint32_t>(cu[1]);
  const int off = cu[2 + blk];
  const uint32_t bits0 = run_bits(0, v0, d1);
  const uint32_t m0 = mine ? bits0 : 0u;
  int cnt = __popc(m0);
  for (int64_t q0 = kWrRun; mine && q0 < Q; q0 += kWrRun) cnt += __popc(taken(q0, d1));
  // exclusive scan of the counts over the block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = cnt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(inc, m, 64);
    if (lane >= m) inc += y;
  }
  if (lane == 63) scan[w] = inc;
  __syncthreads();
  int pre = inc - cnt;
  for (int i = 0; i < w; ++i) pre += scan[i];
  int pos = off + pre;
  for (uint32_t m = m0; m != 0u && pos < k_top; m &= m - 1u)
    out[pos++] = static_cast<int32_t>(b0 + __builtin_ctz(m));
  for (int64_t q0 = kWrRun; mine && q0 < Q; q0 += kWrRun) {
    for (uint32_t m = taken(q0, d1); m != 0u && pos < k_top; m &= m - 1u)
      out[pos++] = static_cast<int32_t>(b0 + q0 + __builtin_ctz(m));
  }
}

// The whole top-k in one launch for units with at most kSmallN candidates:
// one workgroup per unit; thread t loads the scores of its positions [t P,
// t P + P), P <= kSmallP. The unit's range comes from the score kernels'
// partial ranges; the keys then stay in registers and their top-11-bit
// histogram is built in LDS. A boundary bucket of at most kSmallBucket keys
// is collected with its scores and ranked by (score, position); a member's
// key register then holds its slot in the bucket, and the selection (digit
// above, or a member ranked below k_rem) becomes a bit mask per thread,
// whose population is scanned and whose set bits are written in order. A
// larger bucket takes the next two digits from the registers, and refines
// on the score bits the keys dropped when it must (members' scores
// reloaded); the workspace is not used.
constexpr int kSmallP = 32;
constexpr int64_t kSmallN = static_cast<int64_t>(kTopkThreads) * kSmallP;
// units up to this many candidates take the one-launch kernel; larger ones
// the keys, select and write launches, which spread the passes over the
// positions across many compute units
constexpr int64_t kTopkOneLaunchN = kSmallN;
// A copy of x that the compiler cannot relate to x, so that the per-position
// values built on it in one phase are not merged with those of another phase
// (which would keep 32 of them live, or spilled, in between).
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__global__ __launch_bounds__(kTopkThreads) void topk_small_kernel(const int64_t *__restrict__ scores,
                                                                  const unsigned long long *__restrict__ mm,
                                                                  int64_t n, int np, int k_top,
                                                                  int32_t *__restrict__ idx_out) {
  __shared__ TopkShared sh;
  const int unit = blockIdx.x;
  if (k_top == 0) return;
  const int64_t *sc = scores + static_cast<int64_t>(unit) * n;
  int32_t *out = idx_out + static_cast<int64_t>(unit) * k_top;
  const int64_t P = ((n + kTopkThreads - 1) / kTopkThreads + 3) & ~3LL;   // <= kSmallP
  const int64_t j0 = threadIdx.x * P < n ? threadIdx.x * P : n;
  const int64_t j1 = j0 + P < n ? j0 + P : n;
  const int nown = static_cast<int>(j1 - j0);                             // valid: i < nown

  // key[i] of position j0 + i; 0 (no position) for i >= nown. The scores
  // come through a buffer resource over the unit's n scores (loads past the
  // end return 0 and need no per-position mask); the range is the reduction
  // of the score kernels' np partial ranges, by the first wave.
  uint32_t key[kSmallP];
  unsigned long long base;
  int shift, lsh;
  {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int64_t *>(sc), static_cast<short>(0), static_cast<int>(n * 8), 0x00020000);
    const uint32_t vo = opaque_v(static_cast<uint32_t>(j0) * 8u);
    unsigned long long u[kSmallP];
#pragma unroll
    for (int i = 0; i < kSmallP; ++i)
      u[i] = ordered(__builtin_bit_cast(long long, __builtin_amdgcn_raw_buffer_load_b64(rs, vo + 8u * i, 0, 0)));
    clear_whist(sh);
    if (threadIdx.x == 0) sh.bcnt = 0;
    if (threadIdx.x < kSmallBucket) sh.rank[threadIdx.x] = 0;
    unit_range(mm + 2 * static_cast<int64_t>(unit) * np, np, base, shift, lsh, sh.mm);   // ends behind a barrier
    const uint32_t vmask = nown >= 32 ? 0xFFFFFFFFu : (1u << nown) - 1u;
#pragma unroll
    for (int i = 0; i < kSmallP; ++i)
      key[i] = score_key(u[i] - base, shift, lsh) & (0u - ((vmask >> i) & 1u));
  }
  // Plain LDS atomics, one per key: a ballot-merged update (one atomic for
  // the lanes that share the first active lane's bin) costs more
  // instructions per key than the same-bin collisions it saves, even with a
  // crowded first digit (1 x 32K, 8 units: top-k 23.8 -> 19.0 us on N(0, 1)
  // scores, 26.7 -> 22.4 with planted columns, 79 -> 78 with columns that
  // crowd the bulk into a few first digits).
  uint32_t *wh = sh.whist[threadIdx.x >> 7];
#pragma unroll
  for (int i = 0; i < kSmallP; ++i)
    if (key[i] != 0u) atomicAdd(&wh[key[i] >> 21], 1u);
  __syncthreads();
  reduce_whist(sh);
  __syncthreads();
  int k_rem = k_top, eq = 0;
  const uint32_t d1 = static_cast<uint32_t>(find_digit(kBins, &k_rem, &eq, sh));

  if (eq <= kSmallBucket) {                     // eq: from LDS, uniform
    uint32_t memb = 0;                          // bit i: position j0 + i is in the bucket
    const uint32_t jc = opaque_v(static_cast<uint32_t>(j0));
#pragma unroll
    for (int i = 0; i < kSmallP; ++i) {
      if (key[i] != 0u && (key[i] >> 21) == d1) {
        const int slot = atomicAdd(&sh.bcnt, 1);
        sh.bsc[slot] = sc[jc + i];
        sh.bpos[slot] = static_cast<int>(jc + i);
        key[i] = static_cast<uint32_t>(slot);
        memb |= 1u << i;
      }
    }
    __syncthreads();
    rank_bucket(sh, eq);
    // a position outside the range has key 0: digit 0 <= d1, never a member
    auto take = [&](int i) -> bool {
      return ((memb >> i) & 1u) ? sh.rank[key[i]] < k_rem : (key[i] >> 21) > d1;
    };
    uint32_t tmask = 0;                         // bit i: position j0 + i is taken
#pragma unroll
    for (int i = 0; i < kSmallP; ++i) tmask |= static_cast<uint32_t>(take(i)) << i;
    int tot;
    int pos = block_exclusive_scan(__popc(tmask), sh.scan, &tot);
    const uint32_t jw = opaque_v(static_cast<uint32_t>(j0));
    for (; tmask != 0u && pos < k_top; tmask &= tmask - 1u)
      out[pos++] = static_cast<int32_t>(jw + static_cast<uint32_t>(__builtin_ctz(tmask)));
    return;
  }
  // A crowded first digit: the other two digits (bits 10..20, then 0..9)
  // from the keys in registers, giving the key kappa of the k_top-th largest
  // and the number `take` of keys equal to kappa that are taken.
  uint32_t prefix = d1 << 21, pmask = 0x7FFu << 21;
#pragma unroll 1
  for (int ps = 0; ps < 2; ++ps) {
    const int sft = ps == 0 ? 10 : 0;
    const int nbt = ps == 0 ? 11 : 10;
    const uint32_t dm = (1u << nbt) - 1u;
    clear_whist(sh);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSmallP; ++i)
      if (key[i] != 0u && (key[i] & pmask) == prefix) atomicAdd(&wh[(key[i] >> sft) & dm], 1u);
    __syncthreads();
    reduce_whist(sh);
    __syncthreads();
    const int d = find_digit(1 << nbt, &k_rem, &eq, sh);
    prefix |= static_cast<uint32_t>(d) << sft;
    pmask |= dm << sft;
  }
  const uint32_t kappa = prefix;
  int take = k_rem;
  uint32_t sure = 0, tie = 0;                   // bit i: position j0 + i taken for sure / tied
#pragma unroll
  for (int i = 0; i < kSmallP; ++i) {
    sure |= static_cast<uint32_t>(key[i] > kappa) << i;
    tie |= static_cast<uint32_t>(key[i] == kappa) << i;
  }
  if (eq > take && shift > 0) {
    // the keys equal to kappa are not all taken and differ in the low
    // `shift` score bits the keys dropped: select on those bits (their
    // scores reloaded from memory), digit by digit from the top
    const unsigned long long lbits = shift >= 64 ? ~0ull : (1ull << shift) - 1ull;
    const uint32_t jr = opaque_v(static_cast<uint32_t>(j0));
    unsigned long long lowpre = 0, lowmask = 0;
#pragma unroll 1
    for (int top = shift; top > 0; top -= kDigitBits) {
      const int bits = top >= kDigitBits ? kDigitBits : top;
      const int sh2 = top - bits;
      clear_whist(sh);
      __syncthreads();
      for (uint32_t m = tie; m != 0u; m &= m - 1u) {
        const int i = __builtin_ctz(m);
        const unsigned long long lo = (ordered(sc[jr + i]) - base) & lbits;
        if ((lo & lowmask) == lowpre) atomicAdd(&wh[static_cast<uint32_t>(lo >> sh2) & ((1u << bits) - 1u)], 1u);
      }
      __syncthreads();
      reduce_whist(sh);
      __syncthreads();
      int cnt;
      const int d = find_digit(1 << bits, &take, &cnt, sh);
      lowpre |= static_cast<unsigned long long>(d) << sh2;
      lowmask |= static_cast<unsigned long long>((1u << bits) - 1u) << sh2;
    }
    // members above the threshold's low bits are taken; equal ones stay tied
    uint32_t keep = 0;
    for (uint32_t m = tie; m != 0u; m &= m - 1u) {
      const int i = __builtin_ctz(m);
      const unsigned long long lo = (ordered(sc[jr + i]) - base) & lbits;
      if (lo > lowpre) sure |= 1u << i;
      else if (lo == lowpre) keep |= 1u << i;
    }
    tie = keep;
  }
  // keys above kappa (and, after a refinement, members above its low bits)
  // are taken; the tied ones are equal scores, of which the first `take` by
  // position are taken
  int tot;
  const int tie_before = block_exclusive_scan(__popc(tie), sh.scan, &tot);
  uint32_t tmask = sure;
  for (int r = tie_before; tie != 0u && r < take; ++r, tie &= tie - 1u) tmask |= tie & (0u - tie);
  int pos = block_exclusive_scan(__popc(tmask), sh.scan, &tot);
  const uint32_t jw = opaque_v(static_cast<uint32_t>(j0));
  for (; tmask != 0u && pos < k_top; tmask &= tmask - 1u)
    out[pos++] = static_cast<int32_t>(jw + static_cast<uint32_t>(__builtin_ctz(tmask)));
}

// The score kernels have written their partial ranges to topk_mm(tws, units, n).
// skewed: heavy-tailed scores (the attention mass), whose keys crowd a few
// values even at full key resolution; they take the keys, select and write
// launches at every size. Through the one-launch kernel, whose refinement
// reloads the crowded members' scores in every pass, a llama32k mass
// detection on the Llama-shaped synthetic prompt took 149.8 us instead of
// 139.6 (on N(0, 1) scores it gained: 110 -> 103 us).
void launch_topk(hipStream_t st, int units, const int64_t *scores, void *tws, int64_t n, int k_top,
                 int32_t *idx_out, bool skewed = false) {
  const TopkChunks c = topk_chunks(n);
  const TopkWs L = topk_ws(units, n);
  uint8_t *w8 = static_cast<uint8_t *>(tws);
  unsigned long long *mm = reinterpret_cast<unsigned long long *>(w8 + L.mm);
  uint32_t *bh = reinterpret_cast<uint32_t *>(w8 + L.hist);
  uint32_t *keys = reinterpret_cast<uint32_t *>(w8 + L.keys);
  int *ctl = reinterpret_cast<int *>(w8 + L.ctl);
  const int np = topk_partials(n);
  if (n <= kTopkOneLaunchN && !skewed) {
    hipLaunchKernelGGL(topk_small_kernel, dim3(units), dim3(kTopkThreads), 0, st, scores, mm, n, np, k_top, idx_out);
    return;
  }
  const unsigned nb = static_cast<unsigned>(units) * c.nbu;
  hipLaunchKernelGGL(topk_keys_kernel, dim3(nb), dim3(kTkBlock), 0, st, scores, n, c.nbu, c.ch, np, mm, keys, bh);
  hipLaunchKernelGGL(topk_select_kernel, dim3(units), dim3(kTopkThreads), 0, st, scores, keys, bh, mm, n, c.nbu, c.ch,
                     np, k_top, idx_out, ctl);
  hipLaunchKernelGGL(topk_write_kernel, dim3(nb), dim3(kWrThreads), 0, st, keys, ctl, n, c.nbu, c.ch, k_top, idx_out);
}

// ---------------------------------------------------------------- workspace
struct DetWs {
  size_t scores, qs, keys, total;
};
DetWs det_ws(int B, int Hkv, int64_t cand_end) {
  DetWs L{};
  L.scores = 0;
  L.qs = align_up(static_cast<size_t>(B) * Hkv * cand_end * sizeof(int64_t), 256);
  L.keys = align_up(L.qs + static_cast<size_t>(B) * Hkv * 128 * sizeof(double), 256);
  L.total = L.keys + topk_ws(static_cast<int64_t>(B) * Hkv, cand_end).total;
  return L;
}

// Scores from the INT4 cache: c_j = qsum . k_hat_j with k_hat = s c + z
// (fp16 s and z per 32-channel group, codes in the row layout), evaluated
// per group as s (sum_e q_e c_e) + z (sum_e q_e): lane (row, group g) holds
// the group's 32 summed query channels in fp64, loads its 16 code bytes and
// {s, z} word, and the D / 32 lanes of a row add their group terms. A block
// takes 256 rows; every lane issues the loads of all its rows first (one
// row per pass of 256 / (D / 32) rows), then computes, so the block waits
// for one round of loads instead of one per row; the summed query comes
// through LDS once per block. Every product and sum is
// in fp64: exact for queries on the 2^-4 grid within the fp64 range (the
// products are multiples of 2^-28), whatever the order.
template <int D>
__global__ __launch_bounds__(256) void gemv_int4_kernel(const uint8_t *__restrict__ codes,
                                                        const uint32_t *__restrict__ sz,
                                                        const double *__restrict__ qs, int64_t t_cap,
                                                        int64_t cand_end, int chunks_per_unit,
                                                        int64_t *__restrict__ scores,
                                                        unsigned long long *__restrict__ mm) {
  constexpr int NG = D / 32;                // lanes per row, one group each
  constexpr int RPP = 256 / NG;             // rows per pass of the block
  constexpr int CHUNK = 256;
  constexpr int NP = CHUNK / RPP;           // passes
  const int unit = blockIdx.x / chunks_per_unit;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x % chunks_per_unit) * CHUNK;
  const int g = threadIdx.x % NG;
  const int rowi = threadIdx.x / NG;
  uint4 cw[NP];
  uint32_t w[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t r = r0 + rowi + p * RPP;
    if (r < cand_end) {
      const int64_t row = static_cast<int64_t>(unit) * t_cap + r;
      cw[p] = *reinterpret_cast<const uint4 *>(codes + row * (D / 2) + g * 16);
      w[p] = sz[row * NG + g];
    } else {
      cw[p] = make_uint4(0u, 0u, 0u, 0u);
      w[p] = 0u;
    }
  }
  // the unit's summed query, once per block through LDS (lanes of one group
  // read the same words: broadcasts)
  __shared__ double qsh[D];
  if (static_cast<int>(threadIdx.x) < D) qsh[threadIdx.x] = qs[static_cast<int64_t>(unit) * D + threadIdx.x];
  __syncthreads();
  double qv[32];
  double qsum = 0.0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    qv[e] = qsh[g * 32 + e];
    qsum += qv[e];
  }
  unsigned long long mn = ~0ull, mx = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t r = r0 + rowi + p * RPP;
    const uint32_t word[4] = {cw[p].x, cw[p].y, cw[p].z, cw[p].w};
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      acc = fma(qv[e], static_cast<double>((word[e >> 3] >> (4 * (e & 7))) & 0xFu), acc);
    const double s = static_cast<double>(f16_to_f32(w[p] & 0xFFFFu));
    const double z = static_cast<double>(f16_to_f32(w[p] >> 16));
    double part = fma(s, acc, z * qsum);
#pragma unroll
    for (int m = 1; m < NG; m <<= 1) part += __shfl_xor(part, m, 64);
    if (r < cand_end && g == 0) {
      const long long v = __double2ll_rn(part * 65536.0);
      scores[static_cast<int64_t>(unit) * cand_end + r] = v;
      const unsigned long long u = ordered_score(v);
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  block_range_out(mn, mx, mm ? mm + 2 * static_cast<int64_t>(blockIdx.x) : nullptr);
}

// ---------------------------------------------------------------- attention-mass form
// Scores c_j = sum over the unit's query rows rho of softmax_rho(l)_j, the
// attention probability row rho gives key j, l = sm_scale q_rho . k over all
// k_rows keys. Three kernels, each on the column-sum layout above (4 waves,
// two 32-key tiles per wave with their K fragments in registers, the query
// rows staged through LDS 128 at a time):
//  1. mass_stats: per (row, block) partial max (raw logit units) and sum of
//     2^(cs (l - m)) over the block's 256 keys, from S^T = K Q^T (lane = row,
//     registers = keys);
//  2. mass_merge: per row, the partials merged into cs * m and 1 / L;
//  3. mass_cols: per candidate key, sum over rows of 2^(cs l - cs m) / L
//     from S = Q K^T (lane = key, registers = rows), in a fixed order.
// The exponentials make these scores approximate (fp32), not exact.
constexpr float kNegInfF = -__builtin_huge_valf();

template <int D, int DT>
__global__ __launch_bounds__(256) void mass_stats_kernel(const uint16_t *__restrict__ q_acc,
                                                         const uint16_t *__restrict__ k, int Hq, int Hkv,
                                                         int R, int64_t k_rows, int blocks_per_unit,
                                                         float cs, float2 *__restrict__ part) {
  constexpr int KC = D / 16, ROWV = D / 8, PER_T = kStageRows * ROWV / 256;
  __shared__ uint16_t qs[kStageRows][D + kRowPad];
  __shared__ float2 wpart[4][kStageRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int unit = blockIdx.x / blocks_per_unit;
  const int cb = blockIdx.x % blocks_per_unit;
  const int G = Hq / Hkv, b = unit / Hkv, h = unit % Hkv, M = G * R;
  const uint16_t *qrows = q_acc + (static_cast<int64_t>(b) * Hq + h * G) * R * D;
  uint4 kf[2][KC];
  int64_t key0[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    key0[t] = (static_cast<int64_t>(cb) * 8 + wave * 2 + t) * 32;     // first key of the tile
    const int64_t kr = key0[t] + (lane & 31);
    const uint16_t *krow = k + (static_cast<int64_t>(unit) * k_rows + (kr < k_rows ? kr : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      kf[t][kc] = kr < k_rows ? *reinterpret_cast<const uint4 *>(krow + kc * 16 + half * 8)
                              : make_uint4(0u, 0u, 0u, 0u);
  }
  const int stages = (M + kStageRows - 1) / kStageRows;
  for (int st = 0; st < stages; ++st) {
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
      const int idx = e * 256 + threadIdx.x;
      const int row = idx / ROWV, c8 = idx % ROWV;
      const int grow = st * kStageRows + row;
      *reinterpret_cast<uint4 *>(&qs[row][c8 * 8]) =
          grow < M ? *reinterpret_cast<const uint4 *>(qrows + static_cast<int64_t>(grow) * D + c8 * 8)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < kStageRows / 32; ++sub) {
      const uint16_t *qrow = &qs[sub * 32 + (lane & 31)][half * 8];
      float m = kNegInfF, l = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          acc = mfma32<DT>(kf[t][kc], *reinterpret_cast<const uint4 *>(qrow + kc * 16), acc);
        // lane: row sub * 32 + lane % 32; register r: key key0 + 8 (r / 4) + 4 half + r % 4
        float tm = kNegInfF;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = key0[t] + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= k_rows) acc[r] = kNegInfF;
          tm = fmaxf(tm, acc[r]);
        }
        const float mn = fmaxf(m, tm);
        if (mn != kNegInfF) {
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f((acc[r] - mn) * cs);
          l = l * __builtin_amdgcn_exp2f((m - mn) * cs) + sum;
          m = mn;
        }
      }
      // the two halves hold the same row (the other 16 keys of each tile)
      const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
      const float mm = fmaxf(m, mo);
      const float ll = mm == kNegInfF ? 0.f
                                      : l * __builtin_amdgcn_exp2f((m - mm) * cs) +
                                            lo * __builtin_amdgcn_exp2f((mo - mm) * cs);
      if (half == 0) wpart[wave][sub * 32 + lane] = make_float2(mm, ll);
    }
    __syncthreads();
    // merge the 4 waves (fixed order) and write this block's partial per row
    if (threadIdx.x < kStageRows) {
      const int row = st * kStageRows + threadIdx.x;
      float mm = kNegInfF;
#pragma unroll
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, wpart[w][threadIdx.x].x);
      float ll = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float2 v = wpart[w][threadIdx.x];
        if (v.x != kNegInfF) ll += v.y * __builtin_amdgcn_exp2f((v.x - mm) * cs);
      }
      if (row < M) part[(static_cast<int64_t>(unit) * M + row) * blocks_per_unit + cb] = make_float2(mm, ll);
    }
    __syncthreads();
  }
}

// per (unit, row): stats = (cs * m, 1 / L) of the row's softmax over all keys;
// the logits above are raw q . k, so cs = sm_scale * log2(e). One wave per
// row: lanes stride over the row's partials, then a fixed-order wave reduction.
__global__ __launch_bounds__(256) void mass_merge_kernel(const float2 *__restrict__ part, int rows_total,
                                                         int nblk, float cs, float2 *__restrict__ stats) {
  const int r = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows_total) return;                              // wave-uniform
  const float2 *p = part + static_cast<int64_t>(r) * nblk;
  float mm = kNegInfF;
  for (int i = lane; i < nblk; i += 64) mm = fmaxf(mm, p[i].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
  float L = 0.f;
  for (int i = lane; i < nblk; i += 64)
    if (p[i].x != kNegInfF) L += p[i].y * __builtin_amdgcn_exp2f(cs * (p[i].x - mm));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  if (lane == 0) stats[r] = make_float2(cs * mm, L > 0.f ? 1.0f / L : 0.f);
}

template <int D, int DT>
__global__ __launch_bounds__(256) void mass_cols_kernel(const uint16_t *__restrict__ q_acc,
                                                        const uint16_t *__restrict__ k, int Hq, int Hkv, int R,
                                                        int64_t k_rows, int64_t cand_end, int blocks_per_unit,
                                                        float cs, const float2 *__restrict__ stats,
                                                        int64_t *__restrict__ scores,
                                                        unsigned long long *__restrict__ mm) {
  constexpr int KC = D / 16, ROWV = D / 8, PER_T = kStageRows * ROWV / 256;
  __shared__ uint16_t qs[kStageRows][D + kRowPad];
  __shared__ float2 rs[kStageRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int unit = blockIdx.x / blocks_per_unit;
  const int cb = blockIdx.x % blocks_per_unit;
  const int G = Hq / Hkv, b = unit / Hkv, h = unit % Hkv, M = G * R;
  const uint16_t *qrows = q_acc + (static_cast<int64_t>(b) * Hq + h * G) * R * D;
  uint4 kf[2][KC];
  int64_t col[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    col[t] = (static_cast<int64_t>(cb) * 8 + wave * 2 + t) * 32 + (lane & 31);
    const uint16_t *krow = k + (static_cast<int64_t>(unit) * k_rows + (col[t] < cand_end ? col[t] : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      kf[t][kc] = col[t] < cand_end ? *reinterpret_cast<const uint4 *>(krow + kc * 16 + half * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
  }
  float cols[2] = {0.f, 0.f};
  const int stages = (M + kStageRows - 1) / kStageRows;
  for (int st = 0; st < stages; ++st) {
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
      const int idx = e * 256 + threadIdx.x;
      const int row = idx / ROWV, c8 = idx % ROWV;
      const int grow = st * kStageRows + row;
      *reinterpret_cast<uint4 *>(&qs[row][c8 * 8]) =
          grow < M ? *reinterpret_cast<const uint4 *>(qrows + static_cast<int64_t>(grow) * D + c8 * 8)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
    if (threadIdx.x < kStageRows) {
      const int grow = st * kStageRows + threadIdx.x;
      rs[threadIdx.x] = grow < M ? stats[static_cast<int64_t>(unit) * M + grow] : make_float2(0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < kStageRows / 32; ++sub) {
      const uint16_t *arow = &qs[sub * 32 + (lane & 31)][half * 8];
      f32x16 acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 a = *reinterpret_cast<const uint4 *>(arow + kc * 16);
        acc[0] = mfma32<DT>(a, kf[0][kc], acc[0]);
        acc[1] = mfma32<DT>(a, kf[1][kc], acc[1]);
      }
      // lane: key col; register r: row sub * 32 + 8 (r / 4) + 4 half + r % 4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float2 st2 = rs[sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          cols[t] += __builtin_amdgcn_exp2f(fmaf(acc[t][r], cs, -st2.x)) * st2.y;
      }
    }
    __syncthreads();
  }
  unsigned long long mn = ~0ull, mx = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float c = cols[t] + __shfl_xor(cols[t], 32, 64);
    if (half == 0 && col[t] < cand_end) {
      const long long v = __double2ll_rn(static_cast<double>(c) * 4194304.0);   // units of 2^-22
      scores[static_cast<int64_t>(unit) * cand_end + col[t]] = v;
      const unsigned long long u = ordered_score(v);
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  block_range_out(mn, mx, mm ? mm + 2 * static_cast<int64_t>(blockIdx.x) : nullptr);
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
    const size_t need = L.total;
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
  unsigned long long *tmm = k_top > 0 ? topk_mm(static_cast<uint8_t *>(ws) + L.keys, units, cand_end) : nullptr;
  if (cand_end > 0) {
    if (method == HQ_DETECT_MATMUL) {
      const int tiles = static_cast<int>((cand_end + 31) / 32);
      const uint16_t *qa = static_cast<const uint16_t *>(q_acc);
      const uint16_t *kk = static_cast<const uint16_t *>(k);
      const int groups = (tiles + 7) / 8;                    // 256-column groups per unit
      // groups per block: about two blocks per CU over the launch, at most
      // 16. The resident form pays off once a block walks 4 or more groups
      // (16 x 128K: column sums 1291 -> 1148 us); with 2 groups per block
      // (1 x 32K, 8 KV heads) its longer blocks lose (28.9 -> 31.1 us).
      int gpb = static_cast<int>((static_cast<int64_t>(units) * groups) / 512);
      gpb = gpb < 1 ? 1 : (gpb > kResMaxGroups ? kResMaxGroups : gpb);
      // (the resident kernel addresses a unit's candidate rows and scores
      // with 32-bit byte offsets)
      if (D == 128 && (Hq / Hkv) * R <= kResRows && gpb >= 4 && cand_end * D * 2 < (int64_t{1} << 31)) {
        const int rblocks = units * ((groups + gpb - 1) / gpb);
        if (dtype == HQ_BF16)
          hipLaunchKernelGGL((colsum_resident_kernel<128, HQ_BF16>), dim3(rblocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, groups, gpb, scores, tmm);
        else
          hipLaunchKernelGGL((colsum_resident_kernel<128, HQ_F16>), dim3(rblocks), dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, groups, gpb, scores, tmm);
      } else {
        // the 16x16x32 form: 512 columns per block while the grid keeps two
        // blocks per CU, else 256
        const bool wide = static_cast<int64_t>(units) * ((cand_end + 511) / 512) >= 512;
        const int cpb = wide ? 512 : 256;
        const dim3 grid(static_cast<unsigned>(units * ((cand_end + cpb - 1) / cpb)));
        // RES: the unit's query rows fit the two LDS slots at once, and its
        // candidate rows fit a buffer resource's 32-bit byte range
        const bool res = (Hq / Hkv) * R <= 2 * kStageRows && cand_end * D * 2 < (int64_t{1} << 31);
#define HQ_C16R(DD, TT, NN) do { if (res) hipLaunchKernelGGL((mfma16_colsum_kernel<DD, TT, NN, true, 4>), grid, dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, scores, tmm); \
                                 else hipLaunchKernelGGL((mfma16_colsum_kernel<DD, TT, NN, false, 4>), grid, dim3(256), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, scores, tmm); } while (0)
#define HQ_C16(DD, TT) do { if (wide && res && kResWide8) hipLaunchKernelGGL((mfma16_colsum_kernel<DD, TT, 4, true, 8>), grid, dim3(512), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, scores, tmm); \
                            else if (!wide && !res && kStagedNarrow8) hipLaunchKernelGGL((mfma16_colsum_kernel<DD, TT, 2, false, 8>), grid, dim3(512), 0, st, qa, kk, Hq, Hkv, R, k_rows, cand_end, scores, tmm); \
                            else if (wide) HQ_C16R(DD, TT, 8); else HQ_C16R(DD, TT, 4); } while (0)
        if (D == 128) {
          if (dtype == HQ_BF16) HQ_C16(128, HQ_BF16); else HQ_C16(128, HQ_F16);
        } else {
          if (dtype == HQ_BF16) HQ_C16(64, HQ_BF16); else HQ_C16(64, HQ_F16);
        }
#undef HQ_C16
#undef HQ_C16R
      }
    } else {
      double *qs = reinterpret_cast<double *>(static_cast<uint8_t *>(ws) + L.qs);
      switch (dtype) {
        case HQ_F32: hipLaunchKernelGGL(qsum_kernel<HQ_F32>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
        case HQ_BF16: hipLaunchKernelGGL(qsum_kernel<HQ_BF16>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
        default: hipLaunchKernelGGL(qsum_kernel<HQ_F16>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
      }
      const int cpu = static_cast<int>((cand_end + 255) / 256);
      const dim3 grid(static_cast<unsigned>(units * cpu));
#define HQ_GEMV(DD, TT) hipLaunchKernelGGL((gemv_kernel<DD, TT>), grid, dim3(256), 0, st, k, qs, k_rows, cand_end, cpu, scores, tmm)
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
    launch_topk(st, units, scores, static_cast<uint8_t *>(ws) + L.keys, cand_end, k_top, idx_out);
    hq_status s = check_launch("hq_detect_vlines (top-k)");
    if (s != HQ_OK) return s;
  }
  if (ran) *ran = 1;
  clear_error();
  return HQ_OK;
}

extern "C" hq_status hq_detect_vlines_cache(const void *q_new, void *q_acc, hq_dtype dtype, int Hq, int R,
                                            int64_t step, int force, const hq_hybrid_kv *kv,
                                            int64_t cand_end, int k_top, int32_t *idx_out,
                                            int64_t *score_out, int *ran, void *ws, size_t ws_bytes,
                                            void *stream) {
  if (ran) *ran = 0;
  if (!kv) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: null descriptor");
  const int B = kv->B, Hkv = kv->Hkv, D = kv->D;
  if (!dtype_ok(dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: bad dtype");
  if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv)
    return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: bad head counts");
  if (D != 64 && D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_cache: D must be 64 or 128");
  if (kv->group != 32) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_cache: group must be 32");
  if (R < 1 || R > 1024) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: need 1 <= R <= 1024");
  if (step < 0) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: step < 0");
  if (k_top < 0 || cand_end < k_top || cand_end > kv->t_cap || cand_end > kv->T)
    return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: need 0 <= k_top <= cand_end <= min(t_cap, T)");
  if (cand_end > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_cache: cand_end too large");
  if (!q_acc) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: null q_acc");
  const int eb = dtype_bytes(dtype);
  const int slot = static_cast<int>(step % R);
  hipStream_t st = as_stream(stream);
  const bool detect = force || slot == R - 1;
  const DetWs L = det_ws(B, Hkv, cand_end);
  if (detect) {
    if (!kv->k_codes || !kv->k_sz || (k_top > 0 && !idx_out))
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: null INT4 key plane or idx_out");
    if (!ws || ws_bytes < L.total)
      return fail(HQ_ERR_WORKSPACE, "hq_detect_vlines_cache: workspace needs %zu bytes, got %zu", L.total, ws_bytes);
    if (reinterpret_cast<uintptr_t>(kv->k_codes) % 16 || reinterpret_cast<uintptr_t>(kv->k_sz) % 4 ||
        reinterpret_cast<uintptr_t>(q_acc) % 16)
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: misaligned k planes or q_acc");
  }
  if (q_new) {
    if (reinterpret_cast<uintptr_t>(q_new) % 16)
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_cache: q_new must be 16-byte aligned");
    const int rows = B * Hq;
    const int row_bytes = D * eb;
    const int64_t threads = static_cast<int64_t>(rows) * (row_bytes / 16);
    hipLaunchKernelGGL(acc_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint8_t *>(q_new), static_cast<uint8_t *>(q_acc), rows, row_bytes, R,
                       slot);
    hq_status s = check_launch("hq_detect_vlines_cache (accumulate)");
    if (s != HQ_OK) return s;
  }
  if (!detect) { clear_error(); return HQ_OK; }
  int64_t *scores = score_out ? score_out : reinterpret_cast<int64_t *>(static_cast<uint8_t *>(ws) + L.scores);
  const int units = B * Hkv;
  unsigned long long *tmm = k_top > 0 ? topk_mm(static_cast<uint8_t *>(ws) + L.keys, units, cand_end) : nullptr;
  if (cand_end > 0) {
    double *qs = reinterpret_cast<double *>(static_cast<uint8_t *>(ws) + L.qs);
    switch (dtype) {
      case HQ_F32: hipLaunchKernelGGL(qsum_kernel<HQ_F32>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
      case HQ_BF16: hipLaunchKernelGGL(qsum_kernel<HQ_BF16>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
      default: hipLaunchKernelGGL(qsum_kernel<HQ_F16>, dim3(units * (D / 8)), dim3(256), 0, st, q_acc, Hq, Hkv, R, D, qs); break;
    }
    const int cpu = static_cast<int>((cand_end + 255) / 256);
    const dim3 grid(static_cast<unsigned>(units * cpu));
    const uint32_t *szw = reinterpret_cast<const uint32_t *>(kv->k_sz);
    if (D == 128)
      hipLaunchKernelGGL((gemv_int4_kernel<128>), grid, dim3(256), 0, st, kv->k_codes, szw, qs, kv->t_cap, cand_end, cpu, scores, tmm);
    else
      hipLaunchKernelGGL((gemv_int4_kernel<64>), grid, dim3(256), 0, st, kv->k_codes, szw, qs, kv->t_cap, cand_end, cpu, scores, tmm);
    hq_status s = check_launch("hq_detect_vlines_cache (scores)");
    if (s != HQ_OK) return s;
  }
  if (k_top > 0) {
    launch_topk(st, units, scores, static_cast<uint8_t *>(ws) + L.keys, cand_end, k_top, idx_out);
    hq_status s = check_launch("hq_detect_vlines_cache (top-k)");
    if (s != HQ_OK) return s;
  }
  if (ran) *ran = 1;
  clear_error();
  return HQ_OK;
}

namespace hq {
namespace {
struct MassWs {
  size_t scores, part, stats, keys, total;
  int nblk;
};
MassWs mass_ws(int B, int Hq, int Hkv, int R, int64_t k_rows, int64_t cand_end) {
  MassWs L{};
  const int64_t units = static_cast<int64_t>(B) * Hkv;
  const int64_t M = static_cast<int64_t>(Hq / Hkv) * R;
  L.nblk = static_cast<int>((k_rows + 255) / 256);
  L.scores = 0;
  L.part = align_up(static_cast<size_t>(units) * cand_end * sizeof(int64_t), 256);
  L.stats = align_up(L.part + static_cast<size_t>(units) * M * L.nblk * sizeof(float2), 256);
  L.keys = align_up(L.stats + static_cast<size_t>(units) * M * sizeof(float2), 256);
  L.total = L.keys + topk_ws(units, cand_end).total;
  return L;
}
}  // namespace
}  // namespace hq

extern "C" size_t hq_detect_mass_workspace_size(int B, int Hq, int Hkv, int R, int64_t k_rows,
                                                int64_t cand_end) {
  if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv || R < 1 || k_rows < 1 || cand_end < 0) return 0;
  return mass_ws(B, Hq, Hkv, R, k_rows, cand_end).total;
}

extern "C" hq_status hq_detect_vlines_mass(const void *q_new, void *q_acc, hq_dtype dtype, int B, int Hq,
                                           int Hkv, int D, int R, int64_t step, int force, const void *k,
                                           int64_t k_rows, int64_t cand_end, int k_top, float sm_scale,
                                           int32_t *idx_out, int64_t *score_out, int *ran, void *ws,
                                           size_t ws_bytes, void *stream) {
  if (ran) *ran = 0;
  if (dtype != HQ_BF16 && dtype != HQ_F16)
    return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_mass: dtype must be HQ_BF16 or HQ_F16");
  if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: bad head counts");
  if (D != 64 && D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_mass: D must be 64 or 128");
  if (R < 1 || R > 1024) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: need 1 <= R <= 1024");
  if (step < 0) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: step < 0");
  if (k_top < 0 || cand_end < k_top || k_rows < cand_end || k_rows < 1)
    return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: need 0 <= k_top <= cand_end <= k_rows, k_rows >= 1");
  if (k_rows > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_detect_vlines_mass: k_rows too large");
  if (!q_acc) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: null q_acc");
  const int eb = dtype_bytes(dtype);
  const int slot = static_cast<int>(step % R);
  hipStream_t st = as_stream(stream);
  const bool detect = force || slot == R - 1;
  const MassWs L = mass_ws(B, Hq, Hkv, R, k_rows, cand_end);
  if (detect) {
    if (!k || (k_top > 0 && !idx_out)) return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: null k or idx_out");
    if (!ws || ws_bytes < L.total)
      return fail(HQ_ERR_WORKSPACE, "hq_detect_vlines_mass: workspace needs %zu bytes, got %zu", L.total, ws_bytes);
    if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(q_acc) % 16)
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: k and q_acc must be 16-byte aligned");
  }
  if (q_new) {
    if (reinterpret_cast<uintptr_t>(q_new) % 16)
      return fail(HQ_ERR_INVALID_ARG, "hq_detect_vlines_mass: q_new must be 16-byte aligned");
    const int rows = B * Hq;
    const int row_bytes = D * eb;
    const int64_t threads = static_cast<int64_t>(rows) * (row_bytes / 16);
    hipLaunchKernelGGL(acc_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint8_t *>(q_new), static_cast<uint8_t *>(q_acc), rows, row_bytes, R,
                       slot);
    hq_status s = check_launch("hq_detect_vlines_mass (accumulate)");
    if (s != HQ_OK) return s;
  }
  if (!detect) { clear_error(); return HQ_OK; }
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  int64_t *scores = score_out ? score_out : reinterpret_cast<int64_t *>(w8 + L.scores);
  float2 *part = reinterpret_cast<float2 *>(w8 + L.part);
  float2 *stats = reinterpret_cast<float2 *>(w8 + L.stats);
  const int units = B * Hkv;
  unsigned long long *tmm = k_top > 0 ? topk_mm(w8 + L.keys, units, cand_end) : nullptr;
  const int M = (Hq / Hkv) * R;
  const float cs = (sm_scale > 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(D))) * 1.4426950408889634f;
  const uint16_t *qa = static_cast<const uint16_t *>(q_acc);
  const uint16_t *kk = static_cast<const uint16_t *>(k);
  if (cand_end > 0) {
    const int nb1 = L.nblk;
    const int nb3 = static_cast<int>((cand_end + 255) / 256);
#define HQ_MASS(DD, TT)                                                                                  \
  do {                                                                                                   \
    hipLaunchKernelGGL((mass_stats_kernel<DD, TT>), dim3(units * nb1), dim3(256), 0, st, qa, kk, Hq, Hkv, \
                       R, k_rows, nb1, cs, part);                                                        \
    hipLaunchKernelGGL(mass_merge_kernel, dim3((units * M + 3) / 4), dim3(256), 0, st, part,              \
                       units * M, nb1, cs, stats);                                                       \
    hipLaunchKernelGGL((mass_cols_kernel<DD, TT>), dim3(units * nb3), dim3(256), 0, st, qa, kk, Hq, Hkv,  \
                       R, k_rows, cand_end, nb3, cs, stats, scores, tmm);                                 \
  } while (0)
    if (D == 128) {
      if (dtype == HQ_BF16) HQ_MASS(128, HQ_BF16); else HQ_MASS(128, HQ_F16);
    } else {
      if (dtype == HQ_BF16) HQ_MASS(64, HQ_BF16); else HQ_MASS(64, HQ_F16);
    }
#undef HQ_MASS
    hq_status s = check_launch("hq_detect_vlines_mass (scores)");
    if (s != HQ_OK) return s;
  }
  if (k_top > 0) {
    launch_topk(st, units, scores, w8 + L.keys, cand_end, k_top, idx_out, /*skewed=*/true);
    hq_status s = check_launch("hq_detect_vlines_mass (top-k)");
    if (s != HQ_OK) return s;
  }
  if (ran) *ran = 1;
  clear_error();
  return HQ_OK;
}
