// INT4 packing of keys/values and the vertical-line row gather.
//
// Quantizer: "HyQuant ... Explained for Beginners" (aifromscratch.in),
// "How It Works: The Hybrid-Precision Strategy", item 3 -- the quantized
// majority of keys and values is stored in 4 bits. Format (this library's
// reading): per token, 32-channel groups, s = fp16((max - min) / 15),
// z = fp16(min), c = clamp(rint_even((x - z) / s), 0, 15) in fp32 with
// IEEE subtract and correctly rounded divide; s = 0 gives c = 0; a zero
// scale or zero point is stored as +0.
//
// Gather: same page and section, item 1 -- vertical-line tokens keep their
// full-precision keys and values; the gather copies those rows by index into
// the compact 16-bit buffer read by the decode kernel.
//
// This file is compiled with -ffp-contract=off: the quantizer has no
// multiply-add, and keeping contraction off makes the fp32 steps exactly the
// IEEE operations above.
#include <stdio.h>

#include "hq_common.h"
#include "hq_int4.h"

namespace hq {
namespace {

constexpr int kGroup = 32;

// Quantizes one quarter (8 channels) of one (head, row, 32-channel group) of
// x; thread index gid = 4 * item + quarter, and the 4 threads of an item are
// consecutive lanes (a DPP quad) that encode the group together (hq_int4.h).
template <int DT, int LAYOUT>
__device__ __forceinline__ void quantize_quarter(
    uint32_t gid, const void *__restrict__ x, uint32_t n_rows, int D, int64_t x_head_stride,
    int64_t x_row_stride, uint8_t *__restrict__ codes, uint16_t *__restrict__ sz,
    int64_t dst_head_rows, int64_t dst_row0) {
  const int ng = D / kGroup;                  // 2 or 4
  const int q = static_cast<int>(gid & 3u);
  const uint32_t item = gid >> 2;
  const int g = static_cast<int>(item & static_cast<uint32_t>(ng - 1));
  const uint32_t hr = ng == 4 ? (item >> 2) : (item >> 1);
  const uint32_t r = hr % n_rows;
  const uint32_t h = hr / n_rows;

  const int64_t src = static_cast<int64_t>(h) * x_head_stride + static_cast<int64_t>(r) * x_row_stride +
                      g * kGroup + q * 8;
  float v[8];
  load8<DT>(x, src, v);
  _Float16 s16, z16;
  const uint32_t packed = encode_quarter(v, s16, z16);

  const int64_t row = dst_row0 + r;
  const int64_t head_row = static_cast<int64_t>(h) * dst_head_rows + row;
  if constexpr (LAYOUT == HQ_LAYOUT_ROWS) {
    reinterpret_cast<uint32_t *>(codes + head_row * (D / 2) + g * (kGroup / 2))[q] = packed;
  } else {
    // tile u = row / 16 of head h; byte (j, slot(row % 16)) for channel pair
    // j, where each run of 4 rows is stored in the order 0, 2, 1, 3
    const int64_t tile = static_cast<int64_t>(h) * (dst_head_rows / 16) + row / 16;
    const int r16 = static_cast<int>(row % 16);
    const int slot16 = (r16 & ~3) | ((r16 & 1) << 1) | ((r16 >> 1) & 1);
    uint8_t *base = codes + tile * (D / 2) * 16 + slot16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = g * (kGroup / 2) + q * 4 + jj;
      base[j * 16] = static_cast<uint8_t>((packed >> (8 * jj)) & 0xFFu);
    }
  }
  if (q == 0) {
    const uint32_t szw = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
    reinterpret_cast<uint32_t *>(sz)[head_row * (D / kGroup) + g] = szw;
  }
}

// Four threads per (head, row, 32-channel group); the host keeps the thread
// count below 2^31. Items are whole quads, so a quad is either all in range
// or all out.
template <int DT, int LAYOUT>
__global__ __launch_bounds__(256) void quantize_kernel(
    const void *__restrict__ x, int n_heads, int64_t n_rows, int D, int64_t x_head_stride,
    int64_t x_row_stride, uint8_t *__restrict__ codes, uint16_t *__restrict__ sz,
    int64_t dst_head_rows, int64_t dst_row0) {
  const uint32_t total = static_cast<uint32_t>(n_heads) * static_cast<uint32_t>(n_rows) * (D / kGroup) * 4u;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  quantize_quarter<DT, LAYOUT>(gid, x, static_cast<uint32_t>(n_rows), D, x_head_stride, x_row_stride,
                               codes, sz, dst_head_rows, dst_row0);
}

// Values in TILE16, whole tiles only: one wave per (head, tile, 32-channel
// group). Lane (row rr of the tile, quarter q) encodes as quantize_quarter
// does; the codes then pass through LDS so that each tile row (one channel
// pair over the tile's 16 rows, in slot order) leaves as a single 16-byte
// store instead of 16 single-byte stores from different lanes.
template <int DT>
__global__ __launch_bounds__(256) void quantize_tiles_kernel(
    const void *__restrict__ x, int n_heads, int64_t n_tiles, int D, int64_t x_head_stride,
    int64_t x_row_stride, uint8_t *__restrict__ codes, uint16_t *__restrict__ sz,
    int64_t dst_head_rows, int64_t dst_row0, int64_t tile0) {
  __shared__ __align__(16) uint8_t tb[4][16][16];        // [wave][channel pair of the group][slot]
  const int ng = D / kGroup;
  const int wave = static_cast<int>(threadIdx.x >> 6);
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave;   // (head, tile, group)
  if (wid >= static_cast<int64_t>(n_heads) * n_tiles * ng) return;   // wave-uniform
  const int g = static_cast<int>(wid % ng);
  const int64_t ht = wid / ng;
  const int64_t u = tile0 + ht % n_tiles;
  const int64_t h = ht / n_tiles;
  const int rr = lane >> 2, q = lane & 3;
  const int64_t row = u * 16 + rr;
  const int64_t src = h * x_head_stride + (row - dst_row0) * x_row_stride + g * kGroup + q * 8;
  float v[8];
  load8<DT>(x, src, v);
  _Float16 s16, z16;
  const uint32_t packed = encode_quarter(v, s16, z16);
  // each run of 4 rows is stored in the order 0, 2, 1, 3
  const int slot16 = (rr & ~3) | ((rr & 1) << 1) | ((rr >> 1) & 1);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) tb[wave][q * 4 + jj][slot16] = static_cast<uint8_t>((packed >> (8 * jj)) & 0xFFu);
  if (q == 0) {
    const uint32_t szw = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
    reinterpret_cast<uint32_t *>(sz)[(h * dst_head_rows + row) * ng + g] = szw;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane < 16) {
    const uint4 t = *reinterpret_cast<const uint4 *>(&tb[wave][lane][0]);
    uint8_t *tile = codes + (h * (dst_head_rows / 16) + u) * (D / 2) * 16;
    *reinterpret_cast<uint4 *>(tile + (g * 16 + lane) * 16) = t;
  }
}

// Keys (row layout) and values (16-token tiles) of the same rows in one launch:
// the first half of the threads packs K, the second half V.
template <int DT>
__global__ __launch_bounds__(256) void quantize_pair_kernel(
    const void *__restrict__ xk, const void *__restrict__ xv, int n_heads, int64_t n_rows, int D,
    int64_t x_head_stride, int64_t x_row_stride, uint8_t *__restrict__ k_codes,
    uint16_t *__restrict__ k_sz, uint8_t *__restrict__ v_codes, uint16_t *__restrict__ v_sz,
    int64_t dst_head_rows, int64_t dst_row0) {
  const uint32_t total = static_cast<uint32_t>(n_heads) * static_cast<uint32_t>(n_rows) * (D / kGroup) * 4u;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < total) {
    quantize_quarter<DT, HQ_LAYOUT_ROWS>(gid, xk, static_cast<uint32_t>(n_rows), D, x_head_stride,
                                         x_row_stride, k_codes, k_sz, dst_head_rows, dst_row0);
  } else if (gid < 2 * total) {
    quantize_quarter<DT, HQ_LAYOUT_TILE16>(gid - total, xv, static_cast<uint32_t>(n_rows), D,
                                           x_head_stride, x_row_stride, v_codes, v_sz, dst_head_rows,
                                           dst_row0);
  }
}

// One thread per 16-byte chunk of a destination row.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t *__restrict__ src,
                                                     int64_t src_rows, int row_bytes,
                                                     const int32_t *__restrict__ idx, int k,
                                                     int n_heads, uint8_t *__restrict__ dst) {
  const int chunks = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n_heads) * k * chunks;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t hi = gid / chunks;          // h * k + i
  const int64_t h = hi / k;
  const int32_t j = idx[hi];
  uint4 val = make_uint4(0u, 0u, 0u, 0u);
  if (j >= 0 && j < src_rows) {
    val = reinterpret_cast<const uint4 *>(src + (h * src_rows + j) * row_bytes)[c];
  }
  reinterpret_cast<uint4 *>(dst + hi * row_bytes)[c] = val;
}

template <int DT>
void launch_quantize_dt(int layout, dim3 grid, hipStream_t st, const void *x, int n_heads,
                        int64_t n_rows, int D, int64_t xh, int64_t xr, uint8_t *codes,
                        uint16_t *sz, int64_t dhr, int64_t d0) {
  if (layout == HQ_LAYOUT_ROWS) {
    hipLaunchKernelGGL((quantize_kernel<DT, HQ_LAYOUT_ROWS>), grid, dim3(256), 0, st, x,
                       n_heads, n_rows, D, xh, xr, codes, sz, dhr, d0);
    return;
  }
  // TILE16: whole tiles through the tile kernel, the partial tiles at either
  // end (rows [d0, a) and [b, d0 + n_rows)) through the per-byte kernel
  const int64_t end = d0 + n_rows;
  const int64_t a = (d0 + 15) / 16 * 16, b = end / 16 * 16;
  if (b <= a) {
    hipLaunchKernelGGL((quantize_kernel<DT, HQ_LAYOUT_TILE16>), grid, dim3(256), 0, st, x,
                       n_heads, n_rows, D, xh, xr, codes, sz, dhr, d0);
    return;
  }
  const int eb = DT == HQ_F32 ? 4 : 2;
  auto piece = [&](int64_t r0, int64_t r1) {         // rows [r0, r1) by the per-byte kernel
    if (r1 <= r0) return;
    const int64_t threads = 4 * static_cast<int64_t>(n_heads) * (r1 - r0) * (D / kGroup);
    const void *xs = static_cast<const uint8_t *>(x) + (r0 - d0) * xr * eb;
    hipLaunchKernelGGL((quantize_kernel<DT, HQ_LAYOUT_TILE16>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, st, xs, n_heads, r1 - r0, D, xh, xr, codes, sz, dhr, r0);
  };
  piece(d0, a);
  piece(b, end);
  const int64_t n_tiles = (b - a) / 16;
  const int64_t waves = static_cast<int64_t>(n_heads) * n_tiles * (D / kGroup);
  hipLaunchKernelGGL((quantize_tiles_kernel<DT>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st,
                     x, n_heads, n_tiles, D, xh, xr, codes, sz, dhr, d0, a / 16);
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" hq_status hq_quantize_kv(const void *x, hq_dtype x_dtype, int n_heads,
                                    int64_t n_rows, int D, int group, int64_t x_head_stride,
                                    int64_t x_row_stride, uint8_t *codes, uint16_t *sz,
                                    hq_code_layout layout, int64_t dst_head_rows,
                                    int64_t dst_row0, void *stream) {
  if (!dtype_ok(x_dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: bad dtype %d", x_dtype);
  if (layout != HQ_LAYOUT_ROWS && layout != HQ_LAYOUT_TILE16)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: bad layout %d", layout);
  if (group != kGroup) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv: group must be 32");
  if (D != 64 && D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv: D must be 64 or 128");
  if (n_heads < 0 || n_rows < 0 || dst_row0 < 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: negative size");
  if (dst_row0 + n_rows > dst_head_rows)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: rows [%lld, %lld) exceed dst_head_rows %lld",
                (long long)dst_row0, (long long)(dst_row0 + n_rows), (long long)dst_head_rows);
  if (layout == HQ_LAYOUT_TILE16 && dst_head_rows % 16 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: TILE16 needs dst_head_rows %% 16 == 0");
  if (n_heads == 0 || n_rows == 0) { clear_error(); return HQ_OK; }
  if (!x || !codes || !sz) return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: null pointer");
  const int eb = dtype_bytes(x_dtype);
  if ((x_row_stride * eb) % 16 != 0 || (x_head_stride * eb) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sz) % 4 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv: x rows must be 16-byte aligned");
  const int64_t threads = 4 * static_cast<int64_t>(n_heads) * n_rows * (D / kGroup);
  const int64_t blocks = (threads + 255) / 256;
  if (threads > 0x7FFFFF00LL) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv: too many rows for one call");
  dim3 grid(static_cast<unsigned>(blocks));
  hipStream_t st = as_stream(stream);
  switch (x_dtype) {
    case HQ_F32:
      launch_quantize_dt<HQ_F32>(layout, grid, st, x, n_heads, n_rows, D, x_head_stride,
                                 x_row_stride, codes, sz, dst_head_rows, dst_row0);
      break;
    case HQ_BF16:
      launch_quantize_dt<HQ_BF16>(layout, grid, st, x, n_heads, n_rows, D, x_head_stride,
                                  x_row_stride, codes, sz, dst_head_rows, dst_row0);
      break;
    default:
      launch_quantize_dt<HQ_F16>(layout, grid, st, x, n_heads, n_rows, D, x_head_stride,
                                 x_row_stride, codes, sz, dst_head_rows, dst_row0);
      break;
  }
  return check_launch("hq_quantize_kv");
}

extern "C" hq_status hq_gather_rows(const void *src, hq_dtype dtype, int n_heads,
                                    int64_t src_rows, int D, const int32_t *idx, int k, void *dst,
                                    void *stream) {
  if (!dtype_ok(dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_gather_rows: bad dtype %d", dtype);
  if (n_heads < 0 || k < 0 || src_rows < 0 || D <= 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_gather_rows: negative size");
  const int row_bytes = D * dtype_bytes(dtype);
  if (row_bytes % 16 != 0) return fail(HQ_ERR_UNSUPPORTED, "hq_gather_rows: row bytes must be a multiple of 16");
  if (n_heads == 0 || k == 0) { clear_error(); return HQ_OK; }
  if (!src || !idx || !dst) return fail(HQ_ERR_INVALID_ARG, "hq_gather_rows: null pointer");
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return fail(HQ_ERR_INVALID_ARG, "hq_gather_rows: buffers must be 16-byte aligned");
  const int64_t threads = static_cast<int64_t>(n_heads) * k * (row_bytes / 16);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return fail(HQ_ERR_UNSUPPORTED, "hq_gather_rows: too many rows");
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     as_stream(stream), static_cast<const uint8_t *>(src), src_rows, row_bytes,
                     idx, k, n_heads, static_cast<uint8_t *>(dst));
  return check_launch("hq_gather_rows");
}

extern "C" hq_status hq_quantize_kv_pair(const void *xk, const void *xv, hq_dtype x_dtype,
                                         int n_heads, int64_t n_rows, int D, int group,
                                         int64_t x_head_stride, int64_t x_row_stride,
                                         uint8_t *k_codes, uint16_t *k_sz, uint8_t *v_codes,
                                         uint16_t *v_sz, int64_t dst_head_rows, int64_t dst_row0,
                                         void *stream) {
  if (!dtype_ok(x_dtype)) return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: bad dtype %d", x_dtype);
  if (group != kGroup) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv_pair: group must be 32");
  if (D != 64 && D != 128) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv_pair: D must be 64 or 128");
  if (n_heads < 0 || n_rows < 0 || dst_row0 < 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: negative size");
  if (dst_row0 + n_rows > dst_head_rows)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: rows exceed dst_head_rows");
  if (dst_head_rows % 16 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: dst_head_rows must be a multiple of 16");
  if (n_heads == 0 || n_rows == 0) { clear_error(); return HQ_OK; }
  if (!xk || !xv || !k_codes || !k_sz || !v_codes || !v_sz)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: null pointer");
  const int eb = dtype_bytes(x_dtype);
  if ((x_row_stride * eb) % 16 != 0 || (x_head_stride * eb) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(xk) | reinterpret_cast<uintptr_t>(xv) |
       reinterpret_cast<uintptr_t>(k_codes)) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(k_sz) | reinterpret_cast<uintptr_t>(v_sz)) % 4 != 0)
    return fail(HQ_ERR_INVALID_ARG, "hq_quantize_kv_pair: rows must be 16-byte aligned");
  const int64_t threads = 8 * static_cast<int64_t>(n_heads) * n_rows * (D / kGroup);
  const int64_t blocks = (threads + 255) / 256;
  if (threads > 0x7FFFFF00LL) return fail(HQ_ERR_UNSUPPORTED, "hq_quantize_kv_pair: too many rows for one call");
  const dim3 grid(static_cast<unsigned>(blocks));
  hipStream_t st = as_stream(stream);
#define HQ_PAIR(DT_) hipLaunchKernelGGL(quantize_pair_kernel<DT_>, grid, dim3(256), 0, st, xk, xv, n_heads, n_rows, D, x_head_stride, x_row_stride, k_codes, k_sz, v_codes, v_sz, dst_head_rows, dst_row0)
  switch (x_dtype) {
    case HQ_F32: HQ_PAIR(HQ_F32); break;
    case HQ_BF16: HQ_PAIR(HQ_BF16); break;
    default: HQ_PAIR(HQ_F16); break;
  }
#undef HQ_PAIR
  return check_launch("hq_quantize_kv_pair");
}
