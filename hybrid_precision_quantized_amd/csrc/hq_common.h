// Shared host and device helpers of the HyQuant HIP library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq.h"

namespace hq {

// ---------------------------------------------------------------- host side
// Records a message for hq_last_error() and returns `s`.
hq_status fail(hq_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Returns HQ_ERR_HIP with a message if the last launch failed, else HQ_OK.
hq_status check_launch(const char *what);
// Clears the message of the calling thread (called on success).
void clear_error();

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline int dtype_bytes(hq_dtype dt) { return dt == HQ_F32 ? 4 : 2; }
inline bool dtype_ok(int dt) { return dt == HQ_F32 || dt == HQ_BF16 || dt == HQ_F16; }

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}
template <int DT>
__device__ __forceinline__ float load_as_f32(const void *p, int64_t i) {
  if constexpr (DT == HQ_F32) {
    return static_cast<const float *>(p)[i];
  } else if constexpr (DT == HQ_BF16) {
    return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  } else {
    return f16_to_f32(static_cast<const uint16_t *>(p)[i]);
  }
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace hq
