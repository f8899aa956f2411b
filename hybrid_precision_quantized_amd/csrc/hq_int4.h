// INT4 group encoding shared by the quantizer and the prefill pre-pass.
//
// The format: per token, 32-channel groups along head_dim; s = fp16((max -
// min) / 15), z = fp16(min), code c = clamp(rint((x - z) / s), 0, 15), all in
// fp32 with a correctly rounded divide ("HyQuant ... explained simply",
// aifromscratch.in, How It Works: the quantized majority holds 4-bit keys and
// values; the per-group asymmetric format is this library's reading of it).
//
// One group is handled by the 4 lanes of a DPP quad, 8 channels per lane: the
// lanes share the group's min and max through two quad exchanges, then each
// derives the same s and z from the same values with the same instructions
// and codes its own 8 channels.
#pragma once

#include "hq_common.h"

namespace hq {

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// 8 consecutive channels of x starting at element `src`, as fp32
template <int DT>
__device__ __forceinline__ void load8(const void *x, int64_t src, float (&v)[8]) {
  if constexpr (DT == HQ_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + src);
    const float4 f0 = p[0], f1 = p[1];
    v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
    v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + src);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (DT == HQ_BF16) {
        v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
      } else {
        v[2 * j] = f16_to_f32(w[j] & 0xFFFFu);
        v[2 * j + 1] = f16_to_f32(w[j] >> 16);
      }
    }
  }
}

// Encodes this lane's 8 channels; every lane of the quad must call it.
// Returns the fp16 scale and zero and the 8 codes packed as nibbles (channel
// e of the quarter in bits 4e..4e+3).
__device__ __forceinline__ uint32_t encode_quarter(const float (&v)[8], _Float16 &s16, _Float16 &z16) {
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  mn = fminf(mn, quad_dpp<0xB1>(mn));         // quad_perm [1,0,3,2]
  mx = fmaxf(mx, quad_dpp<0xB1>(mx));
  mn = fminf(mn, quad_dpp<0x4E>(mn));         // quad_perm [2,3,0,1]
  mx = fmaxf(mx, quad_dpp<0x4E>(mx));
  // "+ 0.0f" turns a zero of either sign into +0 (IEEE: -0 + +0 = +0).
  const float s32 = (mx - mn) / 15.0f + 0.0f;
  s16 = static_cast<_Float16>(s32);
  z16 = static_cast<_Float16>(mn + 0.0f);
  const float s = static_cast<float>(s16);
  const float z = static_cast<float>(z16);
  // Fast path: q' = (x - z) * rcp(s) is within 2^-18 of the correctly rounded
  // quotient for |q| <= 16 (v_rcp_f32 is good to 1 ulp, the product adds half
  // an ulp; |q| <= 15 (1 + 2^-11) here since s and z are the group's rounded
  // range and minimum). Rounding q' to an integer then agrees with rounding
  // the correctly rounded quotient unless q' lies within 2^-16 of a
  // half-integer; only those elements (exact ties among them) take the IEEE
  // divide. NaN inputs fail the test and take the divide too.
  const float rs = __builtin_amdgcn_rcpf(s);
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c = 0;
    if (s != 0.0f) {
      const float d = v[i] - z;
      const float qf = d * rs;
      float t = __builtin_rintf(qf);
      if (!(0.5f - fabsf(qf - t) > 0x1p-16f)) t = __builtin_rintf(d / s);
      t = fminf(fmaxf(t, 0.0f), 15.0f);
      c = static_cast<uint32_t>(t);
    }
    packed |= c << (4 * i);
  }
  return packed;
}

}  // namespace hq
