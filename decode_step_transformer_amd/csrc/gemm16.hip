// fp16 x fp16 -> fp32 MFMA matrix product for tall products (the prefill
// projections and MLP of the FlexGen layer, [FlexGen] paper notes,
// background section; int4 weights are first expanded to FP16 once per
// layer, as [FlexGen] section 5 prescribes, by k_expand_q4 below).
//
//   y[m][n] = fp16(act(sum_k x[m][k] * wt[n][k]) + res[m][n])
//
// Design (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//  * 512-thread workgroup = 8 waves = 2 waves per SIMD (one wave alone cannot
//    issue MFMAs back to back), one workgroup per CU; tile 256 x 256, waves
//    2 (rows) x 4 (columns), each wave 128 x 64 (32 accumulator tiles).
//  * Both operands go global -> LDS with direct loads (global_load_lds,
//    16 bytes per lane, lane l to slot l of a 1 KB chunk) into a 4-stage ring
//    of 32-deep k-steps (32 KB per stage), three steps ahead of the MFMAs.
//    Rows are 64 bytes; the 16-byte chunk c of row r sits in slot
//    c ^ ((r >> 1) & 3), so fragment reads of 16 consecutive rows hit
//    distinct banks.  The direct loads are issued from inline assembly and
//    their completion is awaited explicitly (vmcnt) before each barrier.
//  * Fragments of the next k-step are read from LDS while the MFMAs of the
//    current one run: after each k-step's barrier the MFMAs start at once,
//    with those reads and the direct loads spread among them.
#include <type_traits>

#include "common.h"
#include "dequant_dev.h"
#include "lds_dma.h"

namespace hp {

namespace {

constexpr int G_BM = 256, G_BN = 256, G_BK = 32, G_NS = 4;
constexpr int G_STAGE = (G_BM + G_BN) * G_BK;  // halves per stage

template <int N, class F>
__device__ __forceinline__ void unroll16(F&& f) {
  if constexpr (N > 0) {
    unroll16<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

struct G16Args {
  const _Float16* A;
  int64_t lda, M;
  const _Float16* W;  // FRAG: fragment-major tiles; else wt[N][K], row stride ldw
  int64_t ldw;
  int K, N, mtiles, ntiles;
  const _Float16* res;
  int64_t ldr;
  int relu;
  _Float16* Y;
  int64_t ldy;
};

// FRAG: the weight is in the fragment-major HP_F16 layout (tile of 16
// columns x 128 inputs = 4 KB, k-step j's 1 KB holding lane L's 8 inputs
// 32 j + 8 (L / 16) .. of column L % 16, the tiles of a k-block adjacent);
// else rows wt[n][k] (the int4 expansion).  Either way a direct load fills
// the same LDS image.
template <bool FRAG>
__global__ __launch_bounds__(512, 1) void k_gemm16(G16Args g) {
  __shared__ __attribute__((aligned(1024))) _Float16 S[G_NS * G_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in an SGPR
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, kq = lane >> 4;

  // tile order: each XCD takes a contiguous run of tiles; runs sweep 4 row
  // tiles per column tile so concurrent tiles share operand slices in L2
  // (the 32 tiles an XCD runs at once: 4 row x 8 column tiles; 2, 8 and 16
  // rows per sweep measured 1-15% slower)
  const int total = g.mtiles * g.ntiles;
  int id = blockIdx.x;
  const int per_xcd = total / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  constexpr int GM = 4;
  const int group = id / (GM * g.ntiles);
  const int first_m = group * GM;
  const int gm = min(GM, g.mtiles - first_m);
  const int mt = first_m + (id % (GM * g.ntiles)) % gm;
  const int nt = (id % (GM * g.ntiles)) / gm;
  const int64_t m0 = (int64_t)mt * G_BM;
  const int n0 = nt * G_BN;

  // direct-load sources: this wave fills A chunks 2w, 2w+1 and B chunks
  // 2w, 2w+1 (16 rows each); lane -> row l/4, slot l%4 holds chunk
  // (l%4) ^ ((row >> 1) & 3)
  const int rin = lane >> 2;
  const int cchunk = (lane & 3) ^ ((rin >> 1) & 3);
  const _Float16* srcA[2];
  const _Float16* srcB[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t m = min(m0 + 16 * (2 * wave + h) + rin, g.M - 1);
    srcA[h] = g.A + m * g.lda + 8 * cchunk;
    if constexpr (FRAG) {
      const int64_t nb = min(n0 + 16 * (2 * wave + h), g.N - 16) / 16;
      srcB[h] = g.W + nb * 2048 + (rin + 16 * cchunk) * 8;
    } else {
      const int64_t n = min(n0 + 16 * (2 * wave + h) + rin, g.N - 1);
      srcB[h] = g.W + n * g.ldw + 8 * cchunk;
    }
  }
  // fragment-major weights: k-step ks is k-step ks % 4 of k-block ks / 4,
  // whose tiles (N / 16 of 4 KB) are adjacent
  auto frag_off = [&](int ks) __attribute__((always_inline)) {
    return (int64_t)(ks >> 2) * (g.N / 16) * 2048 + (ks & 3) * 512;
  };
  const uint32_t sbase = lds_off(S);
  auto issue = [&](int ks, int stage) __attribute__((always_inline)) {
    const int64_t ko = (int64_t)ks * G_BK, kob = FRAG ? frag_off(ks) : ko;
    const uint32_t st = sbase + (uint32_t)stage * G_STAGE * 2;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16(srcA[h] + ko, __builtin_amdgcn_readfirstlane(st + (2 * wave + h) * 1024));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16(srcB[h] + kob, __builtin_amdgcn_readfirstlane(st + G_BM * 64 + (2 * wave + h) * 1024));
  };

  f16x8 fa[2][8], fb[2][4];
  auto read = [&](int buf, int stage) __attribute__((always_inline)) {
    const _Float16* St = S + stage * G_STAGE;
    const int slot = (kq ^ ((r16 >> 1) & 3)) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[buf][i] = *(const f16x8*)(St + (128 * wm + 16 * i + r16) * 32 + slot);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      fb[buf][t] = *(const f16x8*)(St + G_BM * 32 + (64 * wn + 16 * t + r16) * 32 + slot);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KS = g.K / G_BK;
  auto ck = [&](int ks) __attribute__((always_inline)) { return min(ks, KS - 1); };
  // prologue: k-steps 0..3 in flight, fragments of step 0 in registers
  issue(0, 0);
  issue(ck(1), 1);
  issue(ck(2), 2);
  issue(ck(3), 3);
  wait_vm<12>();
  __builtin_amdgcn_s_barrier();
  read(0, 0);

  // step kk: fragments of kk in buffer kk&1; stage (kk+1)&3 must be complete
  // (its loads were issued three steps earlier); stage kk&3 is refilled with
  // step kk+4 once every wave has passed this step's barrier.
  // After the barrier the MFMAs of step kk start at once; the fragment reads
  // of step kk+1 and the four direct loads of step kk+4 are spread over the
  // four groups of 8 MFMAs (two accumulator rows each), so that the matrix
  // cores are not idle while both waves of a SIMD issue memory instructions.
  auto step = [&](int kk, auto cur_) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_)::value;
    wait_vm<8, 0>();  // this wave's reads of stage kk are done, and its loads of kk+1
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int64_t ko = (int64_t)ck(kk + 4) * G_BK, kob = FRAG ? frag_off(ck(kk + 4)) : ko;
    const uint32_t stg = sbase + (uint32_t)(kk & 3) * G_STAGE * 2;
    const _Float16* St = S + ((kk + 1) & 3) * G_STAGE;
    const int slot = (kq ^ ((r16 >> 1) & 3)) * 8;
    unroll16<4>([&](auto c_) {
      constexpr int c = decltype(c_)::value;
      const _Float16* Sa = St + (128 * wm + 32 * c + r16) * 32 + slot;
      fa[cur ^ 1][2 * c] = *(const f16x8*)Sa;
      fa[cur ^ 1][2 * c + 1] = *(const f16x8*)(Sa + 16 * 32);
      fb[cur ^ 1][c] = *(const f16x8*)(St + G_BM * 32 + (64 * wn + 16 * c + r16) * 32 + slot);
      unroll16<2>([&](auto i_) {
        constexpr int i = 2 * c + decltype(i_)::value;
        unroll16<4>([&](auto t_) {
          constexpr int t = decltype(t_)::value;
          acc[i][t] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[cur][t], fa[cur][i], acc[i][t], 0, 0, 0);
        });
      });
      unroll16<3>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (c < 2)
        dma16(srcA[c] + ko, __builtin_amdgcn_readfirstlane(stg + (2 * wave + c) * 1024));
      else
        dma16(srcB[c - 2] + kob,
              __builtin_amdgcn_readfirstlane(stg + G_BM * 64 + (2 * wave + c - 2) * 1024));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  int kk = 0;
  for (; kk + 2 <= KS; kk += 2) {
    step(kk, std::integral_constant<int, 0>());
    step(kk + 1, std::integral_constant<int, 1>());
  }
  if (kk < KS) step(kk, std::integral_constant<int, 0>());
  wait_vm<0>();

  // epilogue: lane holds rows m0 + 128 wm + 16 i + r16, columns
  // n0 + 64 wn + 16 t + 4 kq .. +3
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + 128 * wm + 16 * i + r16;
    if (m >= g.M) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + 64 * wn + 16 * t + 4 * kq;
      if (n >= g.N) continue;
      f32x4 v = acc[i][t];
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

// Expands a packed int4 weight (see hp_mat) into wt[n][k] binary16:
// fp16(c * scale + min) with one rounding.  One thread per 16-byte chunk of
// the packed layout = 32 consecutive k of one output column.
__global__ __launch_bounds__(256) void k_expand_q4(const u32x4* __restrict__ packed,
                                                   const _Float16* __restrict__ scale,
                                                   const _Float16* __restrict__ minv, int K, int N,
                                                   _Float16* __restrict__ wt, int64_t ldw) {
  const DqConst dq{0x000F000Fu, 0x00F000F0u, in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
  const int KB = K / 128;
  const int64_t total = (int64_t)(N / 16) * KB * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int L = (int)(idx & 63);
    const int64_t tile = idx >> 6;
    const int kb = (int)(tile % KB), nb = (int)(tile / KB);
    const int n = 16 * nb + (L & 15);
    const int k0 = 128 * kb + 32 * (L >> 4);
    const u32x4 c = packed[idx];
    const _Float16* sp = scale + (int64_t)(n >> 6) * K + k0;
    const _Float16* mp = minv + (int64_t)(n >> 6) * K + k0;
    _Float16* out = wt + (int64_t)n * ldw + k0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 s = *(const u32x4*)(sp + 8 * j);
      const u32x4 m = *(const u32x4*)(mp + 8 * j);
      *(f16x8*)(out + 8 * j) = dequant8(c[j], s, m, dq);
    }
  }
}

}  // namespace

hp_status launch_gemm16(const void* x, int64_t ldx, const void* wt, int64_t ldw, int k, int n,
                        int64_t M, const void* res, int64_t ldr, bool relu, void* y, int64_t ldy,
                        hipStream_t st) {
  if (M == 0) return HP_OK;
  G16Args a;
  a.A = (const _Float16*)x;
  a.lda = ldx;
  a.M = M;
  a.W = (const _Float16*)wt;
  a.ldw = ldw;
  a.K = k;
  a.N = n;
  a.mtiles = (int)cdiv(M, G_BM);
  a.ntiles = (int)cdiv(n, G_BN);
  a.res = (const _Float16*)res;
  a.ldr = ldr;
  a.relu = relu ? 1 : 0;
  a.Y = (_Float16*)y;
  a.ldy = ldy;
  Prof prof("gemm_f16_tiled", st);
  const dim3 grid((unsigned)(a.mtiles * a.ntiles));
  if (ldw == 0)
    hipLaunchKernelGGL(k_gemm16<true>, grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(k_gemm16<false>, grid, dim3(512), 0, st, a);
  return launch_ok("k_gemm16");
}

hp_status launch_expand_q4(const hp_mat& w, void* wt, int64_t ldw, hipStream_t st) {
  const int64_t total = (int64_t)(w.n / 16) * (w.k / 128) * 64;
  const int blocks = (int)std::min<int64_t>(cdiv(total, 256), 65536);
  Prof prof("expand_q4", st);
  hipLaunchKernelGGL(k_expand_q4, dim3(blocks), dim3(256), 0, st, (const u32x4*)w.data,
                     (const _Float16*)w.scale, (const _Float16*)w.minv, w.k, w.n, (_Float16*)wt, ldw);
  return launch_ok("k_expand_q4");
}

}  // namespace hp
