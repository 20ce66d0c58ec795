// Skinny int4 products of the decode step: y = act(x·w) + res with x of at
// most 144 rows and w in the packed group-wise int4 layout ([FlexGen] paper
// notes, section 5: int4 weights in groups of 64 along the output channels,
// converted back to FP16 right before the product; background section: the
// projections and MLP products are x·w).
//
// Design (gfx950, v_mfma_f32_16x16x32_f16, one 512-thread workgroup per CU):
//  * The workgroup owns 256 output columns for one k-range (split-K); its 8
//    waves are 4 column groups (64 columns = one int4 group, 4 subtiles of
//    16) times 2 row halves, so two waves share every SIMD and one wave's
//    MFMAs overlap the other's dequantisation.
//  * Activations, packed codes and group scales/mins all reach LDS through
//    direct loads (global_load_lds, no registers): activations in 2 stages
//    (double-buffered, L2-resident), codes and scales in 4 stages, so weight
//    bytes are requested 3 k-blocks before use.  Waits are explicit vmcnt
//    counts: in every k-block each wave issues the next activation block
//    first and then the weight block three ahead, so waiting for the
//    activations leaves the last weight block in flight.
//  * Activation rows are 256 B with 16-byte chunks XOR-swizzled by row, so
//    the fragment reads of 16 consecutive rows hit distinct banks.
//  * Codes are expanded in registers with the magic-exponent trick and one
//    packed FMA with scale and min (a single rounding).
//  * Split partials go to fp32 scratch, summed in split order by
//    k_splitk_reduce (so a row's result never depends on M).
#include <type_traits>

#include "common.h"
#include "dequant_dev.h"
#include "lds_dma.h"

namespace hp {

namespace {

constexpr int XS = 2;               // activation stages
constexpr int WS = 4;               // code / scale stages
constexpr int WBYTES = 16 * 1024;   // 16 subtiles x (64 lanes x 16 B)
constexpr int SBYTES = 4 * 512;     // 4 groups x (128 scale + 128 min halves)

template <int N, class F>
__device__ __forceinline__ void unr(F&& f) {
  if constexpr (N > 0) {
    unr<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

struct DqArgs {
  const _Float16* A;
  int64_t lda;
  int M, K, N, splits, ntiles;
  const uint8_t* B;  // packed codes: [n/16][k/128][64 lanes][16 B]
  const _Float16* scale;
  const _Float16* minv;
  const _Float16* res;
  int64_t ldr;
  int relu;
  _Float16* Y;
  int64_t ldy;
  float* P;  // split partials [split][M][N] or null
};

// One wave: row tiles [rt0, rt0 + TM) of the staged SR rows, 64 columns of
// column group wcol.
template <int TM, int SR>
__device__ __forceinline__ void dq_wave(const DqArgs& g, uint8_t* lds, int wave, int wcol, int rt0,
                                        int nt, int split) {
  constexpr int XB = SR * 256;  // bytes per activation stage
  constexpr int NX = SR / 32;   // activation loads per wave per k-block
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int KB = g.K / 128;
  const int kb0 = split * KB / g.splits, kb1 = (split + 1) * KB / g.splits;
  const int nb = kb1 - kb0;
  uint8_t* Xl = lds;
  uint8_t* Wl = lds + XS * XB;
  uint8_t* Sl = Wl + WS * WBYTES;
  const uint32_t xbase = lds_off(Xl), wbase = lds_off(Wl), sbase = lds_off(Sl);

  // ---- direct-load sources of this lane ----
  // activations: load p covers rows 32 p + 4 wave + (lane >> 4); LDS slot
  // (lane & 15) of a row holds chunk slot ^ (row & 15).  Rows past M reload
  // row M-1 (never stored).
  const _Float16* xsrc[NX];
  unr<NX>([&](auto p_) {
    constexpr int p = decltype(p_)::value;
    const int row = 32 * p + 4 * wave + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    xsrc[p] = g.A + (int64_t)min(row, g.M - 1) * g.lda + 8 * c;
  });
  // codes: subtiles 2 wave and 2 wave + 1 of the workgroup's 16 (columns
  // past N reload the last subtile, never stored)
  const uint8_t* wsrc[2];
  unr<2>([&](auto h_) {
    constexpr int h = decltype(h_)::value;
    const int n16 = min(nt * 16 + 2 * wave + h, g.N / 16 - 1);
    wsrc[h] = g.B + ((int64_t)n16 * KB * 64 + lane) * 16;
  });
  // scales (even waves) or mins (odd waves) of group wave >> 1, lanes 0-15
  const int gi = min(nt * 4 + (wave >> 1), g.N / 64 - 1);
  const _Float16* ssrc = ((wave & 1) ? g.minv : g.scale) + (int64_t)gi * g.K + 8 * (lane & 15);

  auto blk = [&](int i) __attribute__((always_inline)) { return kb0 + min(i, nb - 1); };
  auto issue_x = [&](int i) __attribute__((always_inline)) {
    const int kb = blk(i);
    const uint32_t base = xbase + (i & 1) * XB + wave * 1024;
    unr<NX>([&](auto p_) {
      constexpr int p = decltype(p_)::value;
      dma16(xsrc[p] + kb * 128, __builtin_amdgcn_readfirstlane(base + p * 8192));
    });
  };
  auto issue_ws = [&](int i) __attribute__((always_inline)) {
    const int kb = blk(i);
    const uint32_t wb = wbase + (i & 3) * WBYTES + 2 * wave * 1024;
    dma16(wsrc[0] + (int64_t)kb * 1024, __builtin_amdgcn_readfirstlane(wb));
    dma16(wsrc[1] + (int64_t)kb * 1024, __builtin_amdgcn_readfirstlane(wb + 1024));
    const uint32_t sb = sbase + (i & 3) * SBYTES + (wave >> 1) * 512 + (wave & 1) * 256;
    if (lane < 16) dma16(ssrc + kb * 128, __builtin_amdgcn_readfirstlane(sb));
  };

  // ---- fragments ----
  const DqConst dq{0x000F000Fu, 0x00F000F0u, in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
  f32x4 acc[TM][4];
  unr<TM>([&](auto i_) {
    unr<4>([&](auto t_) { acc[decltype(i_)::value][decltype(t_)::value] = f32x4{0.f, 0.f, 0.f, 0.f}; });
  });
  // Operands of the expansion: the 4 subtiles' codes of a whole k-block
  // (one 16-byte read each, read during the previous block) and per k-step
  // scale/min pairs (read one k-step ahead); activation fragments are read
  // one k-step before their MFMAs.  Buffers alternate with the parity of the
  // k-step (scales, fragments) and of the k-block (codes).
  struct SM {
    u32x4 sv, mv;
  };
  SM sa, sb;
  u32x4 ca[4], cb[4];
  f16x8 xa[TM], xb[TM], wa[4], wb[4];
  // k-step j of a k-block: lane quarter kq contributes k = 32 kq + 8 j .. +7
  auto read_x = [&](f16x8 (&x)[TM], int xs, int j) __attribute__((always_inline)) {
    const uint8_t* base = Xl + xs * XB + (16 * rt0 + r16) * 256 + 16 * ((4 * kq + j) ^ r16);
    unr<TM>([&](auto i_) {
      constexpr int i = decltype(i_)::value;
      x[i] = *(const f16x8*)(base + i * 16 * 256);
    });
  };
  auto read_s = [&](SM& o, int wsg, int j) __attribute__((always_inline)) {
    const uint8_t* sp = Sl + wsg * SBYTES + wcol * 512 + 64 * kq + 16 * j;
    o.sv = *(const u32x4*)sp;
    o.mv = *(const u32x4*)(sp + 256);
  };
  auto read_c = [&](u32x4 (&c)[4], int wsg) __attribute__((always_inline)) {
    const uint8_t* cp = Wl + wsg * WBYTES + 4 * wcol * 1024 + lane * 16;
    unr<4>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      c[t] = *(const u32x4*)(cp + t * 1024);
    });
  };
  auto make_w = [&](f16x8 (&w)[4], const u32x4 (&c)[4], const SM& o, auto j_)
      __attribute__((always_inline)) {
    constexpr int j = decltype(j_)::value;
    unr<4>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      w[t] = dequant8(c[t][j], o.sv, o.mv, dq);
    });
  };
  auto mma = [&](const f16x8 (&w)[4], const f16x8 (&x)[TM]) __attribute__((always_inline)) {
    unr<TM>([&](auto i_) {
      constexpr int i = decltype(i_)::value;
      unr<4>([&](auto t_) {
        constexpr int t = decltype(t_)::value;
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[t], x[i], acc[i][t], 0, 0, 0);
      });
    });
  };
  // issue order in one k-step: NR LDS reads first, then each MFMA followed by
  // VPM VALU instructions (the expansion for the next k-step)
  constexpr int VPM = (56 + 4 * TM - 1) / (4 * TM);
  auto interleave = [&](auto nr_) __attribute__((always_inline)) {
    unr<decltype(nr_)::value>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
    unr<4 * TM>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // One k-block i with codes in `cur`; the codes of block i+1 go to `nxt`.
  // At entry wa = expanded k-step 0 of block i and sb = its k-step 1 scales.
  auto block = [&](int i, const u32x4 (&cur)[4], u32x4 (&nxt)[4]) __attribute__((always_inline)) {
    const int xs = i & 1, wsg = i & 3, wsg1 = (i + 1) & 3;
    // activations of block i (and codes of block i+1) are in LDS for every
    // wave; every wave is done with block i-1
    wait_vm<3, 0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_x(xa, xs, 0);
    issue_x(i + 1);
    issue_ws(i + 3);
    __builtin_amdgcn_sched_barrier(0);
    read_x(xb, xs, 1);
    read_s(sa, wsg, 2);
    mma(wa, xa);
    make_w(wb, cur, sb, I1());
    interleave(std::integral_constant<int, TM + 2>());
    __builtin_amdgcn_sched_barrier(0);
    read_x(xa, xs, 2);
    read_s(sb, wsg, 3);
    read_c(nxt, wsg1);
    mma(wb, xb);
    make_w(wa, cur, sa, I2());
    interleave(std::integral_constant<int, TM + 6>());
    __builtin_amdgcn_sched_barrier(0);
    read_x(xb, xs, 3);
    read_s(sa, wsg1, 0);
    mma(wa, xa);
    make_w(wb, cur, sb, I3());
    interleave(std::integral_constant<int, TM + 2>());
    __builtin_amdgcn_sched_barrier(0);
    read_s(sb, wsg1, 1);
    mma(wb, xb);
    make_w(wa, nxt, sa, I0());
    interleave(std::integral_constant<int, 2>());
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: codes/scales of blocks 0..2 and activations of block 0
  issue_ws(0);
  issue_ws(1);
  issue_x(0);
  issue_ws(2);
  wait_vm<6 + NX>();  // block 0's codes and scales (own loads)
  __builtin_amdgcn_s_barrier();
  read_c(ca, 0);
  read_s(sa, 0, 0);
  read_s(sb, 0, 1);
  make_w(wa, ca, sa, I0());

  // pairs of blocks, so that the code buffers swap roles without copies
  int i = 0;
  for (; i + 2 <= nb; i += 2) {
    block(i, ca, cb);
    block(i + 1, cb, ca);
  }
  if (i < nb) block(i, ca, cb);
  wait_vm<0>();  // no direct load may still target LDS when the group ends

  const int n_wave = nt * 256 + wcol * 64;
  if (n_wave >= g.N) return;
  // ---- epilogue: lane holds rows 16 (rt0 + i) + r16, columns n .. n+3 ----
  unr<TM>([&](auto i_) {
    constexpr int i = decltype(i_)::value;
    const int m = 16 * (rt0 + i) + r16;
    if (m >= g.M) return;
    unr<4>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      const int n = n_wave + 16 * t + 4 * kq;
      f32x4 v = acc[i][t];
      if (g.P) {
        *(f32x4*)(g.P + ((int64_t)split * g.M + m) * g.N + n) = v;
        return;
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
    });
  });
}

template <int TA, int TB>
__global__ __launch_bounds__(512, 1) void k_gemm_dq(DqArgs g) {
  constexpr int SR = 32 * ((TA + TB + 1) / 2);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[XS * SR * 256 + WS * (WBYTES + SBYTES)];
  // workgroups on one XCD (id % 8) take a contiguous run of (split, column
  // tile) pairs, split-major, so they share activation k-slices in L2
  const int total = g.ntiles * g.splits;
  int id = blockIdx.x;
  const int per_xcd = total / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  const int split = id / g.ntiles, nt = id % g.ntiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4)
    dq_wave<TA, SR>(g, lds, wave, wave, 0, nt, split);
  else
    dq_wave<TB, SR>(g, lds, wave, wave - 4, TA, nt, split);
}

}  // namespace

hp_status launch_gemm_dq(const void* x, int64_t ldx, const hp_mat& w, int64_t M, const void* res,
                         int64_t ldr, bool relu, void* y, int64_t ldy, int splits, float* partials,
                         hipStream_t st) {
  DqArgs a;
  a.A = (const _Float16*)x;
  a.lda = ldx;
  a.M = (int)M;
  a.K = w.k;
  a.N = w.n;
  a.splits = splits;
  a.ntiles = (int)cdiv(w.n, 256);
  a.B = (const uint8_t*)w.data;
  a.scale = (const _Float16*)w.scale;
  a.minv = (const _Float16*)w.minv;
  a.res = (const _Float16*)res;
  a.ldr = ldr;
  a.relu = relu ? 1 : 0;
  a.Y = (_Float16*)y;
  a.ldy = ldy;
  a.P = splits > 1 ? partials : nullptr;
  const dim3 grid((unsigned)(a.ntiles * splits));
  const int T = (int)cdiv(M, 16);
  Prof prof("gemm_q4_skinny", st);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, a); };
  switch (T) {
    case 2: go(k_gemm_dq<1, 1>); break;
    case 3: go(k_gemm_dq<2, 1>); break;
    case 4: go(k_gemm_dq<2, 2>); break;
    case 5: go(k_gemm_dq<3, 2>); break;
    case 6: go(k_gemm_dq<3, 3>); break;
    case 7: go(k_gemm_dq<4, 3>); break;
    case 8: go(k_gemm_dq<4, 4>); break;
    default: go(k_gemm_dq<5, 4>); break;
  }
  return launch_ok("k_gemm_dq");
}

}  // namespace hp
