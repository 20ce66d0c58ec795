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
//
// The code of x is clamp(rint(t), 0, 15) with t = fl(fl(fl(x - min) / r) * 15)
// in binary32 (correctly rounded division).  That division costs about ten
// instructions, so each code is first taken from t' = fl(fl(x - min) * y),
// y = 15 * rcp(r) (rcp within 1 ulp): t and t' both lie within 3 ulp(15) of
// 15 (x - min) / r, so |t - t'| < 6e-6 and, whenever t' is farther than
// 2^-15 from a half-integer, rint(t') = rint(t).  Only the rare elements
// near a rounding boundary (and NaN, or infinite inputs) take the exact
// division; the result is bit-identical to evaluating t for every element.
// 16-byte load of data read once (non-temporal: it should not displace
// reusable lines in the caches).
__device__ __forceinline__ uint4 stream_load16(const uint4* p) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 v = __builtin_nontemporal_load((const v4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int CTRL>
__device__ __forceinline__ float quant_dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t quant_group8(uint4 raw, uint32_t& smw) {
#pragma clang fp contract(off)
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffff));
    v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  // the group's 8 lanes: quad_perm [1,0,3,2], [2,3,0,1], then the mirror
  // within each half row of 8 lanes
  mn = fminf(mn, quant_dpp<0xB1>(mn));
  mx = fmaxf(mx, quant_dpp<0xB1>(mx));
  mn = fminf(mn, quant_dpp<0x4E>(mn));
  mx = fmaxf(mx, quant_dpp<0x4E>(mx));
  mn = fminf(mn, quant_dpp<0x141>(mn));
  mx = fmaxf(mx, quant_dpp<0x141>(mx));
  // -0 counts as +0: only the stored min can tell them apart (the codes and
  // max - min come out the same either way)
  mn = mn + 0.0f;
  const float r = mx - mn;
  uint32_t even = 0, odd = 0;  // codes 0, 2, 4, 6 and 1, 3, 5, 7, one per byte
  if (r > 0.0f) {
    const float y = 15.0f * __builtin_amdgcn_rcpf(r);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = v[i] - mn;
      float c = __builtin_rintf(a * y);
      if (!(__builtin_fabsf(a * y - c) < 0.5f - 0x1p-15f)) {
        const float t = a / r * 15.0f;  // the defining evaluation
        c = fminf(fmaxf(__builtin_rintf(t), 0.0f), 15.0f);
      }
      if (i & 1)
        odd = __builtin_amdgcn_cvt_pk_u8_f32(c, i >> 1, odd);
      else
        even = __builtin_amdgcn_cvt_pk_u8_f32(c, i >> 1, even);
    }
    smw = f16_bits_of(r / 15.0f) | (f16_bits_of(mn) << 16);
  } else {
    smw = __builtin_isfinite(mn) ? (f16_bits_of(mn) << 16) : 0u;
  }
  return even | (odd << 4);
}

}  // namespace hp
