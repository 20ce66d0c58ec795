// int4 -> binary16 expansion shared by the GEMM kernels (group-wise
// asymmetric int4 weights of [FlexGen] section 5: value = code * scale + min,
// one rounding).
#pragma once

#include "common.h"

namespace hp {

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Expands one dword of 8 int4 codes (nibble order of the packed layout:
// pair p = (nibble p, nibble p+4) gives k-offsets (2p, 2p+1)) to 8 binary16
// values c * scale + min, given the 4 scale pairs and 4 min pairs.
// A nibble inserted at mantissa bits 0..3 of a half under the exponent of
// 1024, or at bits 4..7 under the exponent of 64, has weight exactly 1, so
// the half reads as magic + c and one packed subtraction gives the exact
// integer c.  Pairs 0 and 1 sit at bits 0..3 and 4..7 of each half already;
// pairs 2 and 3 after one shift by 8.  The final packed FMA rounds once, as
// the dequantiser's definition requires.  Masks and magic patterns arrive in
// registers so that each insert is one v_and_or_b32.
struct DqConst {
  uint32_t mask0, mask1;    // 0x000F000F, 0x00F000F0
  uint32_t magic0, magic1;  // 0x64006400 (1024), 0x54005400 (64)
};
// (a & m) | b with b & m == 0: one v_and_or_b32 (m in an SGPR, b in a VGPR:
// a VOP3 instruction may read only one SGPR)
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | b; }
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
  return r;
}
__device__ __forceinline__ f16x2 fma2(f16x2 c, uint32_t s, uint32_t m) {
  return __builtin_elementwise_fma(c, __builtin_bit_cast(f16x2, s), __builtin_bit_cast(f16x2, m));
}
__device__ __forceinline__ f16x8 dequant8(uint32_t w, u32x4 s, u32x4 m, const DqConst& q) {
  const f16x2 o0 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const f16x2 o1 = {(_Float16)64.0f, (_Float16)64.0f};
  const uint32_t w8 = w >> 8;
  const f16x2 c0 = __builtin_bit_cast(f16x2, bfi(q.mask0, w, q.magic0)) - o0;
  const f16x2 c1 = __builtin_bit_cast(f16x2, bfi(q.mask1, w, q.magic1)) - o1;
  const f16x2 c2 = __builtin_bit_cast(f16x2, bfi(q.mask0, w8, q.magic0)) - o0;
  const f16x2 c3 = __builtin_bit_cast(f16x2, bfi(q.mask1, w8, q.magic1)) - o1;
  return as_f16x8(u32x4{__builtin_bit_cast(uint32_t, fma2(c0, s[0], m[0])),
                        __builtin_bit_cast(uint32_t, fma2(c1, s[1], m[1])),
                        __builtin_bit_cast(uint32_t, fma2(c2, s[2], m[2])),
                        __builtin_bit_cast(uint32_t, fma2(c3, s[3], m[3]))});
}

}  // namespace hp
