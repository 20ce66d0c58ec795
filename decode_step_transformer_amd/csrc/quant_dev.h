// Device-side int4 group-64 coder shared by the quantiser and the KV append
// kernels ([FlexGen] paper notes, section 5, group-wise quantization).
// Eight consecutive lanes (aligned to 8) hold one group of 64 binary16
// values, 8 per lane, as one 16-byte vector.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace hp {

__device__ __forceinline__ uint32_t f16_bits_of(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// Returns this lane's 8 codes packed as nibbles (element e at bits 4e) and,
// through smw, the group's {scale, min} as two binary16 in one dword
// (scale in the low half).  All 8 lanes of the group must be active.
__device__ __forceinline__ uint32_t quant_group8(uint4 raw, uint32_t& smw) {
#pragma clang fp contract(off)
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffff)) + 0.0f;
    v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16)) + 0.0f;
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  const float r = mx - mn;
  uint32_t word = 0;
  if (r > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = (v[i] - mn) / r * 15.0f;
      const float q = fminf(fmaxf(rintf(t), 0.0f), 15.0f);
      word |= (uint32_t)q << (4 * i);
    }
    smw = f16_bits_of(r / 15.0f) | (f16_bits_of(mn) << 16);
  } else {
    smw = __builtin_isfinite(mn) ? (f16_bits_of(mn) << 16) : 0u;
  }
  return word;
}

}  // namespace hp
