// Building blocks of the streaming decode-attention kernels ([FlexGen]
// paper notes, background section: the decode step's softmax(q K^T / sqrt(d)) V
// over the cached rows; section 5: the cache is int4 groups of 64 along the
// hidden dimension, value = code * scale + min).
//
// A wave works on one query of one (request, head).  Every lane reads 16
// consecutive bytes of a cache row, so LPR lanes cover a row and one load
// instruction covers RPI consecutive rows:
//  * scores: codes become halves off + c with a shift and one and-or; every
//    code reads 64 + c and the offsets cancel against the accumulator's start
//    value -64 sum(q); the group scale and min are factored out:
//    s = sum_g scale_g (q . c)_g + min_g (sum q)_g;
//  * values: sum_t p_t v_t = sum_t (p_t scale_t) c_t + sum_t p_t min_t, the
//    first term with one mixed-precision FMA per code (binary16 off + c,
//    fp32 weight and sum), the offsets removed once at the end with the sum
//    of the weights.
#pragma once

#include <math.h>

#include "common.h"
#include "dequant_dev.h"

namespace hp {

// ------------------------------------------------------------ reductions
__device__ __forceinline__ f16x2 h2_of(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Cross-lane moves on the DPP path (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
constexpr int DPP_ROR = 0x120;        // + 1..15: rotate right within a row of 16 lanes

// Lane pairs l, l ^ 16 and l, l ^ 32 through gfx950's row swaps
// (v_permlane16_swap, v_permlane32_swap: vector registers only, no LDS
// round trip).  Given the same value as both operands, a swap returns the
// pair's two values, the lower lane's first, in both lanes of the pair.
__device__ __forceinline__ void pair16(float v, float& lo, float& hi) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}
// v + v of lane l ^ 16 (resp. l ^ 32), the same bits in both lanes
__device__ __forceinline__ float sum_xor16(float v) {
  float a, b;
  pair16(v, a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float v) {
  float a, b;
  pair32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float max_xor16(float v) {
  float a, b;
  pair16(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float v) {
  float a, b;
  pair32(v, a, b);
  return fmaxf(a, b);
}

// sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16): every lane gets its group's sum
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
  if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
  if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp<DPP_MIRROR>(v);
  return v;
}
// sum over the lanes congruent modulo N (N = 1, 2, 4, 8, 16): every lane gets the total
template <int N>
__device__ __forceinline__ float strided_sum(float v) {
  if constexpr (N <= 1) v += dpp<DPP_ROR + 1>(v);
  if constexpr (N <= 2) v += dpp<DPP_ROR + 2>(v);
  if constexpr (N <= 4) v += dpp<DPP_ROR + 4>(v);
  if constexpr (N <= 8) v += dpp<DPP_ROR + 8>(v);
  // (the row swaps measured no faster here: these kernels keep the vector
  // units busy with the int4 expansion, and the LDS pipe is otherwise idle)
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
// wave-uniform maximum: DPP within each row of 16 lanes, then the four rows
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  const int b = __builtin_bit_cast(int, v);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}

// ------------------------------------------------------- lane geometry
template <int D, bool Q4>
struct DecShape {
  static constexpr int LPR = Q4 ? D / 32 : D / 8;
  static constexpr int RPI = 64 / LPR;
  static constexpr int RB = Q4 ? D / 2 : 2 * D;  // bytes per cache row
  static constexpr int NA = Q4 ? 32 : 8;         // value dims per lane
  static constexpr int G = D / 64;               // int4 groups per row
};

// U rows' share of this lane: 16 code bytes per row and (Q4) the row's
// scale/min pair of this lane's group
template <int U, bool Q4>
struct DecPart {
  u32x4 c[U];
  uint32_t sm[Q4 ? U : 1];
};

// ------------------------------------------------------------- query
// This lane's slice of the query, paired in the order the codes expand
// (Q4: pair p of dword j = dims (8j+p, 8j+p+4)).  In the score an expanded
// code reads 64 + c; the accumulator starts at -64 sum(q), so it ends at
// sum(c * q).  The small offset keeps the cancelled magnitude, and so the
// fp32 rounding of the running sum, near that of sum(c * q) itself.
template <int D, bool Q4>
struct DecQuery {
  static constexpr int NQ = Q4 ? 16 : 4;
  f16x2 q2[NQ];
  float corr = 0.f, qsum = 0.f;

  // qp: the query's dims handled by this lane ((Q4 ? 32 : 8) of them)
  __device__ __forceinline__ void load(const _Float16* qp) {
    using S = DecShape<D, Q4>;
#pragma unroll
    for (int j = 0; j < NQ / 4; ++j) {
      const f16x8 qh = *(const f16x8*)(qp + 8 * j);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (Q4) {
          q2[4 * j + p] = f16x2{qh[p], qh[p + 4]};
          corr += 64.f * ((float)qh[p] + (float)qh[p + 4]);
          qsum += (float)qh[p] + (float)qh[p + 4];
        } else {
          q2[4 * j + p] = f16x2{qh[2 * p], qh[2 * p + 1]};
        }
      }
    }
    if constexpr (Q4) qsum = group_sum<S::LPR / S::G>(qsum);  // sum of q over this lane's group
  }
};

// q . k for the row whose 16-byte slice (and scale/min pair) this lane
// holds; every lane of the row gets the whole score.
template <int D, bool Q4>
__device__ __forceinline__ float row_score(const u32x4& c, uint32_t smw, const DecQuery<D, Q4>& Q,
                                           const DqConst& dq) {
  using S = DecShape<D, Q4>;
  float t;
  if constexpr (Q4) {
    t = -Q.corr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // every pair at bits 4..7 / 20..23 under the exponent of 64
      const uint32_t w = c[j];
      t = __builtin_amdgcn_fdot2(h2_of(bfi(dq.mask1, w << 4, dq.magic1)), Q.q2[4 * j + 0], t, false);
      t = __builtin_amdgcn_fdot2(h2_of(bfi(dq.mask1, w, dq.magic1)), Q.q2[4 * j + 1], t, false);
      t = __builtin_amdgcn_fdot2(h2_of(bfi(dq.mask1, w >> 4, dq.magic1)), Q.q2[4 * j + 2], t, false);
      t = __builtin_amdgcn_fdot2(h2_of(bfi(dq.mask1, w >> 8, dq.magic1)), Q.q2[4 * j + 3], t, false);
    }
    t = group_sum<S::LPR / S::G>(t);  // sum(c * q) over the group
    const f16x2 sm = h2_of(smw);
    t = fmaf((float)sm[0], t, (float)sm[1] * Q.qsum);
    if constexpr (S::G == 2) t += dpp<DPP_XOR2>(t);
  } else {
    t = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) t = __builtin_amdgcn_fdot2(h2_of(c[j]), Q.q2[j], t, false);
    t = group_sum<S::LPR>(t);
  }
  return t;
}

// ------------------------------------------------------------- values
// sum_t p_t v_t over this lane's rows for its NA dims (see the header).
template <int D, bool Q4>
struct DecAcc {
  static constexpr int NA = DecShape<D, Q4>::NA;
  float acc[NA];
  float bsum = 0.f, pm = 0.f;  // Q4: sum of the weights p*scale, sum of p*min (this group)

  __device__ __forceinline__ DecAcc() {
#pragma unroll
    for (int e = 0; e < NA; ++e) acc[e] = 0.f;
  }
  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int e = 0; e < NA; ++e) acc[e] *= alpha;
    bsum *= alpha;
    pm *= alpha;
  }
  // U rows with weights p[u]
  template <int U>
  __device__ __forceinline__ void add(const DecPart<U, Q4>& V, const float (&p)[U],
                                      const DqConst& dq) {
    if constexpr (Q4) {
      // weights p * scale stay in fp32: each code meets its row's weight in
      // one mixed-precision FMA (binary16 code, fp32 weight and sum)
      float bw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f16x2 sm = h2_of(V.sm[u]);
        bw[u] = p[u] * (float)sm[0];
        bsum += bw[u];
        pm = fmaf(p[u], (float)sm[1], pm);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = V.c[u][j], x8 = x >> 8;
          const f16x2 c04 = h2_of(bfi(dq.mask0, x, dq.magic0));   // codes 8j, 8j+4 (+1024)
          const f16x2 c15 = h2_of(bfi(dq.mask1, x, dq.magic1));   // codes 8j+1, 8j+5 (+64)
          const f16x2 c26 = h2_of(bfi(dq.mask0, x8, dq.magic0));  // codes 8j+2, 8j+6 (+1024)
          const f16x2 c37 = h2_of(bfi(dq.mask1, x8, dq.magic1));  // codes 8j+3, 8j+7 (+64)
          float* A = acc + 8 * j;
          A[0] = fmaf((float)c04[0], bw[u], A[0]);
          A[4] = fmaf((float)c04[1], bw[u], A[4]);
          A[1] = fmaf((float)c15[0], bw[u], A[1]);
          A[5] = fmaf((float)c15[1], bw[u], A[5]);
          A[2] = fmaf((float)c26[0], bw[u], A[2]);
          A[6] = fmaf((float)c26[1], bw[u], A[6]);
          A[3] = fmaf((float)c37[0], bw[u], A[3]);
          A[7] = fmaf((float)c37[1], bw[u], A[7]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f16x8 vh = __builtin_bit_cast(f16x8, V.c[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf((float)vh[e], p[u], acc[e]);
      }
    }
  }
  // Adds up the row slots (lanes with the same dims) and, on the lanes of
  // row slot 0, writes out = acc / l for this lane's dims.  l_lane: the sum
  // of this lane's row weights (each row's weight counted by its LPR lanes).
  __device__ __forceinline__ void finish(float l_lane, int rho, _Float16* o) {
    constexpr int LPR = DecShape<D, Q4>::LPR;
    const float l = strided_sum<1>(l_lane) * (1.0f / LPR);
#pragma unroll
    for (int e = 0; e < NA; ++e) acc[e] = strided_sum<LPR>(acc[e]);
    if constexpr (Q4) {
      bsum = strided_sum<LPR>(bsum);
      pm = strided_sum<LPR>(pm);
    }
    if (rho == 0) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int j = 0; j < NA / 8; ++j) {
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[8 * j + e];
          if constexpr (Q4) v = v - ((e & 1) ? 64.f : 1024.f) * bsum + pm;
          y[e] = (_Float16)(v * inv);
        }
        *(f16x8*)(o + 8 * j) = y;
      }
    }
  }
};

}  // namespace hp
