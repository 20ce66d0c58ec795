// Dequant-fused MFMA matrix product y = act(x·w) + res for the FlexGen layer
// ([FlexGen] paper notes, background section: Q/K/V/O projections and the
// two MLP products are all x·w; section 5: int4 weights are converted back
// to FP16 before the product).
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//  * A workgroup is 4 waves and owns a BM x 256 output tile (BM = 16 TM);
//    wave w owns output columns [64 w, 64 w + 64) = one int4 group, as 4
//    16-column subtiles, for all BM rows.
//  * The activation tile x[BM][128] of each k-block is staged through LDS
//    (double-buffered, rows padded by 16 B) and shared by the 4 waves.
//  * Weight fragments go straight from HBM to registers: in the packed
//    layout one 16-column subtile of one 128-deep k-block is 1 KB, 16 B per
//    lane, already in MFMA fragment order; int4 codes are expanded with the
//    1024-offset binary16 trick and one packed FMA with the group's scale and
//    min (a single rounding, the same value the oracle's dequantiser gives).
//  * MFMA operand A is the weight fragment (16 output columns), operand B the
//    activation fragment (16 rows), so each lane ends with 4 consecutive
//    output columns of one row: 8-byte stores.
//  * Skinny products (M <= 144, the decode step) split k over workgroups;
//    partial sums go to fp32 scratch and a second kernel adds them in split
//    order, so the result depends only on (k, n), never on M.
#include "common.h"

namespace hp {

constexpr int BK = 128;        // k-block (one packed q4 tile in depth)
constexpr int LDS_ROW = 136;   // halves per staged activation row (128 + 8 pad)
constexpr int SKINNY_M = 144;  // largest M handled as one row tile with split-k

__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

// Expands one dword of 8 int4 codes (nibble order of the packed layout) to 8
// binary16 values c * scale + min, given the 4 scale pairs and 4 min pairs.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint4 s, uint4 m) {
  const uint32_t sp[4] = {s.x, s.y, s.z, s.w};
  const uint32_t mp[4] = {m.x, m.y, m.z, m.w};
  const f16x2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
  uint32_t out[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u = ((w >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
    const f16x2 c = __builtin_bit_cast(f16x2, u) - off;  // exact small integers
    const f16x2 y = __builtin_elementwise_fma(c, __builtin_bit_cast(f16x2, sp[p]),
                                              __builtin_bit_cast(f16x2, mp[p]));
    out[p] = __builtin_bit_cast(uint32_t, y);
  }
  return as_f16x8(make_uint4(out[0], out[1], out[2], out[3]));
}

struct GemmArgs {
  const _Float16* A;
  int64_t lda, M;
  const void* B;
  const _Float16* scale;
  const _Float16* minv;
  int K, N, kb_per_split, mtiles;
  const _Float16* res;
  int64_t ldr;
  int relu;
  _Float16* Y;
  int64_t ldy;
  float* P;  // split partials [split][M][N] or null
};

template <int TM, bool Q4>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  constexpr int BM = 16 * TM;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KB = g.K / BK;
  const int ntiles = (g.N + 255) / 256;

  // tile order: workgroups on the same XCD (id % 8) take a contiguous run of
  // tiles, and runs sweep 4 row tiles at a time so that concurrently running
  // tiles share activation and weight k-slices in L2.
  const int total = g.mtiles * ntiles;
  int id = blockIdx.x;
  const int per_xcd = total / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  constexpr int GM = 4;
  const int group = id / (GM * ntiles);
  const int first_m = group * GM;
  const int gm = min(GM, g.mtiles - first_m);
  const int mt = first_m + (id % (GM * ntiles)) % gm;
  const int nt = (id % (GM * ntiles)) / gm;

  const int64_t m0 = (int64_t)mt * BM;
  const int n_wave = nt * 256 + wave * 64;
  const bool wave_on = n_wave < g.N;
  const int split = blockIdx.y;
  const int kb0 = split * g.kb_per_split, kb1 = kb0 + g.kb_per_split;

  // ---- activation tile loader: TM 16-byte chunks per thread ----
  uint4 areg[TM];
  auto load_a = [&](int kb) {
#pragma unroll
    for (int c = 0; c < TM; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk >> 4, col = (chunk & 15) * 8;
      const int64_t m = m0 + row;
      areg[c] = (m < g.M) ? *(const uint4*)(g.A + m * g.lda + (int64_t)kb * BK + col)
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int c = 0; c < TM; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk >> 4, col = (chunk & 15) * 8;
      *(uint4*)(&As[buf][row * LDS_ROW + col]) = areg[c];
    }
  };

  // ---- weight fragment loader (double-buffered in registers) ----
  const int kq = lane >> 4, r16 = lane & 15;
  const int grp = n_wave >> 6;
  struct Raw {
    uint4 c[Q4 ? 4 : 16];  // Q4: codes per subtile; F16: 4 chunks per subtile
    uint4 sc[Q4 ? 4 : 1], mn[Q4 ? 4 : 1];
  };
  auto load_b = [&](Raw& R, int kb) {
    if (!wave_on) return;
    if constexpr (Q4) {
      const uint4* P = (const uint4*)g.B;
#pragma unroll
      for (int t = 0; t < 4; ++t) R.c[t] = P[((int64_t)((n_wave >> 4) + t) * KB + kb) * 64 + lane];
      const int64_t so = (int64_t)grp * g.K + (int64_t)kb * BK + 32 * kq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        R.sc[j] = *(const uint4*)(g.scale + so + 8 * j);
        R.mn[j] = *(const uint4*)(g.minv + so + 8 * j);
      }
    } else {
      const _Float16* W = (const _Float16*)g.B;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4* p = (const uint4*)(W + (int64_t)(n_wave + 16 * t + r16) * g.K +
                                        (int64_t)kb * BK + 32 * kq);
#pragma unroll
        for (int j = 0; j < 4; ++j) R.c[4 * t + j] = p[j];
      }
    }
  };

  f32x4 acc[TM][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Raw& R, int cur) {
    if (!wave_on) return;
    const _Float16* Ab = &As[cur][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 wf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (Q4) {
          const uint4 c = R.c[t];
          const uint32_t w = j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
          wf[t] = dequant8(w, R.sc[j], R.mn[j]);
        } else {
          wf[t] = as_f16x8(R.c[4 * t + j]);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const f16x8 xf = *(const f16x8*)(Ab + (16 * i + r16) * LDS_ROW + 32 * kq + 8 * j);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[t], xf, acc[i][t], 0, 0, 0);
      }
    }
  };

  // one k-block: prefetch the next activation tile and weight fragments,
  // multiply this block, then publish the next activation tile
  auto step = [&](int kb, const Raw& cur_b, Raw& next_b) {
    const int cur = (kb - kb0) & 1;
    const bool more = kb + 1 < kb1;
    if (more) {
      load_a(kb + 1);
      load_b(next_b, kb + 1);
    }
    compute(cur_b, cur);
    if (more) store_a(cur ^ 1);
    __syncthreads();
  };

  Raw b0, b1;
  load_a(kb0);
  store_a(0);
  load_b(b0, kb0);
  __syncthreads();
  for (int kb = kb0; kb < kb1; kb += 2) {
    step(kb, b0, b1);
    if (kb + 1 < kb1) step(kb + 1, b1, b0);
  }

  if (!wave_on) return;
  // ---- epilogue: lane holds rows m = m0 + 16 i + r16, columns n .. n+3 ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + 16 * i + r16;
    if (m >= g.M) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n_wave + 16 * t + 4 * kq;
      f32x4 v = acc[i][t];
      if (g.P) {
        *(f32x4*)(g.P + ((int64_t)split * g.M + m) * g.N + n) = v;
        continue;
      }
      if (g.relu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.0f);
      }
      if (g.res) {
        const f16x4 r = *(const f16x4*)(g.res + m * g.ldr + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += (float)r[e];
      }
      f16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (_Float16)v[e];
      *(f16x4*)(g.Y + m * g.ldy + n) = o;
    }
  }
}

// Sums split-k partials in split order, then applies the epilogue.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ P, int splits,
                                                       int64_t M, int N,
                                                       const _Float16* __restrict__ res,
                                                       int64_t ldr, int relu,
                                                       _Float16* __restrict__ Y, int64_t ldy) {
  const int64_t quads = M * (N / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const int64_t m = q / (N / 4);
    const int n = (int)(q % (N / 4)) * 4;
    f32x4 v = *(const f32x4*)(P + m * N + n);
    for (int s = 1; s < splits; ++s) v += *(const f32x4*)(P + ((int64_t)s * M + m) * N + n);
    if (relu) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.0f);
    }
    if (res) {
      const f16x4 r = *(const f16x4*)(res + m * ldr + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += (float)r[e];
    }
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (_Float16)v[e];
    *(f16x4*)(Y + m * ldy + n) = o;
  }
}

// Split factor for skinny products: a function of (k, n) only.
static int split_for(int32_t k, int32_t n) {
  const int KB = k / BK;
  const int ntiles = (int)cdiv(n, 256);
  const int want = (int)cdiv(512, ntiles);
  for (int d = 1; d <= KB && d <= 16; ++d)
    if (KB % d == 0 && d >= want) return d;
  int best = 1;
  for (int d = 1; d <= KB && d <= 16; ++d)
    if (KB % d == 0) best = d;
  return best;
}

size_t gemm_ws_bytes(int64_t M, int32_t k, int32_t n) {
  if (M > SKINNY_M || M <= 0) return 0;
  const int s = split_for(k, n);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)n * sizeof(float) : 0;
}

template <int TM>
static void launch_tm(const GemmArgs& a, bool q4, dim3 grid, hipStream_t st) {
  const bool skinny = a.mtiles == 1 && TM <= 9 && a.M <= SKINNY_M;
  Prof prof(q4 ? (skinny ? "gemm_q4_skinny" : "gemm_q4_tiled")
               : (skinny ? "gemm_f16_skinny" : "gemm_f16_tiled"), st);
  if (q4)
    hipLaunchKernelGGL((k_gemm<TM, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<TM, false>), grid, dim3(256), 0, st, a);
}

hp_status launch_gemm(const void* x, int64_t ldx, const hp_mat& w, int64_t M, const void* res,
                      int64_t ldr, bool relu, void* y, int64_t ldy, void* ws, hipStream_t st) {
  if (M == 0) return HP_OK;
  GemmArgs a;
  a.A = (const _Float16*)x;
  a.lda = ldx;
  a.M = M;
  a.B = w.data;
  a.scale = (const _Float16*)w.scale;
  a.minv = (const _Float16*)w.minv;
  a.K = w.k;
  a.N = w.n;
  a.res = (const _Float16*)res;
  a.ldr = ldr;
  a.relu = relu ? 1 : 0;
  a.Y = (_Float16*)y;
  a.ldy = ldy;
  a.P = nullptr;
  const bool q4 = w.fmt == HP_Q4;
  const int KB = w.k / BK;
  const int ntiles = (int)cdiv(w.n, 256);
  if (M <= SKINNY_M) {
    const int TM = (int)cdiv(M, 16);
    const int splits = split_for(w.k, w.n);
    a.kb_per_split = KB / splits;
    a.mtiles = 1;
    if (splits > 1) a.P = (float*)ws;
    const dim3 grid(ntiles, splits);
    switch (TM) {
      case 1: launch_tm<1>(a, q4, grid, st); break;
      case 2: launch_tm<2>(a, q4, grid, st); break;
      case 3: launch_tm<3>(a, q4, grid, st); break;
      case 4: launch_tm<4>(a, q4, grid, st); break;
      case 5: launch_tm<5>(a, q4, grid, st); break;
      case 6: launch_tm<6>(a, q4, grid, st); break;
      case 7: launch_tm<7>(a, q4, grid, st); break;
      case 8: launch_tm<8>(a, q4, grid, st); break;
      default: launch_tm<9>(a, q4, grid, st); break;
    }
    hp_status s = launch_ok("k_gemm");
    if (s != HP_OK || splits == 1) return s;
    const int64_t quads = M * (w.n / 4);
    const int blocks = (int)std::min<int64_t>(cdiv(quads, 256), 8192);
    Prof prof("gemm_splitk_reduce", st);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, st, (const float*)ws, splits,
                       M, w.n, (const _Float16*)res, ldr, a.relu, (_Float16*)y, ldy);
    return launch_ok("k_splitk_reduce");
  }
  a.kb_per_split = KB;
  a.mtiles = (int)cdiv(M, 128);
  const dim3 grid((unsigned)(a.mtiles * ntiles), 1);
  launch_tm<8>(a, q4, grid, st);
  return launch_ok("k_gemm");
}

}  // namespace hp
