// The fp8 E4M3 encoder of the cache writes: bf16 rows times 1 / scale,
// saturated to the format's finite range and rounded by the hardware
// conversion, NaN kept as the NaN code. The cache writes (cache_ops.hip) and
// the decode that stores its step's token (decode.hip) share it, so both
// produce the same codes.
#pragma once
#include "device_common.h"

namespace kvp {

// bf16 -> fp8 E4M3 code of x * inv: fp32 product, saturated to the
// format's finite range (+-448), then the hardware conversion (round to
// nearest, ties to even). A NaN input is handled by fp8_pack4.
__device__ __forceinline__ float fp8_prep(uint32_t bf16_bits, float inv) {
  const float x = __builtin_bit_cast(float, bf16_bits << 16) * inv;
  return fminf(fmaxf(x, -448.f), 448.f);
}

// Four bf16 values (two dwords) -> four codes. A NaN input (bf16 exponent
// all ones, mantissa non-zero) is stored as the NaN code S.1111.111 with the
// input's sign, whatever the clamp above made of it: E4M3 keeps NaN.
__device__ __forceinline__ uint32_t fp8_pack4(uint32_t w0, uint32_t w1,
                                              float inv) {
  int r = 0;
  r = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prep(w0 & 0xFFFF, inv),
                                      fp8_prep(w0 >> 16, inv), r, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prep(w1 & 0xFFFF, inv),
                                      fp8_prep(w1 >> 16, inv), r, true);
  uint32_t out = (uint32_t)r;
  const uint32_t h[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if ((h[i] & 0x7FFFu) > 0x7F80u) {
      const uint32_t nan_code = 0x7Fu | ((h[i] >> 8) & 0x80u);
      out = (out & ~(0xFFu << (8 * i))) | (nan_code << (8 * i));
    }
  }
  return out;
}

// Reciprocal of the scale of head h: per-head scales (device array) when
// given, else the tensor's. 1.f / x is correctly rounded in HIP device code.
__device__ __forceinline__ float fp8_inv(const float* scales, float inv,
                                         int64_t h) {
  return scales ? 1.f / scales[h] : inv;
}

}  // namespace kvp
