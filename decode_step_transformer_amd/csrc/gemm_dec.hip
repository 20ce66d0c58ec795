// Skinny int4 products of the decode step: y = act(x·w) + res with x of 1 to
// 144 rows and w in the packed group-wise int4 layout ([FlexGen] paper
// notes, section 5: int4 weights in groups of 64 along the output channels,
// converted back to FP16 right before the product; background section: the
// projections and MLP products are x·w).
//
// Design (gfx950, v_mfma_f32_16x16x32_f16, one 512-thread workgroup per CU):
//  * The workgroup owns 256 output columns for one k-range (split-K).  Its
//    8 waves are 4 column groups (64 columns = one int4 group, 4 subtiles
//    of 16) times 2 k-step halves: the two waves on a SIMD (w and w + 4)
//    hold all row tiles of the same 64 columns, wave w takes k-steps 0, 1 of
//    each 128-deep k-block and wave w + 4 k-steps 2, 3.  Every weight element
//    is expanded once per workgroup, and each activation fragment read from
//    LDS feeds 4 MFMAs.  The two partial sums are added through LDS at the
//    end (a fixed order).
//  * Activations, packed codes and group scales/mins all reach LDS through
//    direct loads (global_load_lds, no registers): activations in 2 stages
//    (L2-resident), codes and scales in 4 stages, so weight bytes are
//    requested 3 k-blocks before use.  Waits are explicit vmcnt counts.
//  * LDS is the scarce resource (every byte of activations is read by four
//    waves), so the per-block reads are kept to one 8-byte read of codes per
//    subtile and one dword of scales/mins per lane; the 8 scale and 8 min
//    pairs a lane needs per k-step come from the lanes of its row of 16 by
//    DPP broadcast.  Activation rows are 256 B with 16-byte chunks XOR-
//    swizzled by row (a fragment read hits every bank once).
//  * Codes are expanded in registers with the magic-exponent trick and one
//    packed FMA with scale and min (a single rounding).
//  * Split partials go to fp32 scratch in the kernel's own tile-major order
//    (each store instruction writes 1 KB contiguous) and are summed in split
//    order by k_dq_reduce (so a row's result never depends on M).
#include <type_traits>

#include "common.h"
#include "dequant_dev.h"
#include "lds_dma.h"

namespace hp {

namespace {

constexpr int XS = 2;              // activation stages
constexpr int WS = 4;              // code / scale stages
constexpr int WBYTES = 16 * 1024;  // 16 subtiles x (64 lanes x 16 B)
constexpr int SCH = 288;           // one scale or min chunk (128 halves), padded
constexpr int SBYTES = 8 * SCH;    // 4 groups x (scale chunk, min chunk)

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

// Chunk swizzle of an activation row r (16-byte chunk c sits in slot
// c ^ xswz(r & 15)): a fragment read puts 16 rows x 4 lane quarters of
// chunks on LDS banks; with the bits of r reordered, the rows of one parity
// use one of each pair of slots {x, x ^ 4}, so lane quarters 0 and 1 (and 2
// and 3) never meet in a bank (the plain r ^ c put them 2-way in conflict,
// measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int xswz(int r) { return ((r >> 1) & 3) | ((r & 1) << 2) | (r & 8); }

// Lane n of each row of 16 lanes, to every lane of that row.
template <int n>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + n, 0xF, 0xF, false);
}

// One wave: column group wave & 3, all TM row tiles, k-steps 2 PH and
// 2 PH + 1 of every k-block.
//
// Per wave the pipeline runs over its own steps (two per k-block): at the
// start of a step the wave holds the step's activations and expanded
// weights; during the step's MFMAs it expands the next step's weights and,
// after the 4 MFMAs of each row tile, reads that tile's activations of the
// next step into the registers just released.  Codes and scales of both of
// the wave's steps of a block are read once, in its second step of the
// previous block (after the k-block barrier that wave passes at the start of
// that step, when its activations of the block are in registers: direct
// loads of the next block have landed; the activations two blocks ahead and
// the weights three blocks ahead are issued).
template <int TM, int PH>
__device__ __forceinline__ void dq_pair(const DqArgs& g, uint8_t* lds, int wave, int nt,
                                        int split) {
  constexpr int SR = 16 * TM;                          // staged rows
  constexpr int XB = SR * 256;                         // bytes per activation stage
  constexpr int NX = PH == 0 ? (TM + 1) / 2 : TM / 2;  // activation loads per block
  constexpr int NWS = 3;  // code (2) and scale-or-min (1) loads per block
  constexpr int J0 = 2 * PH;
  const int wcol = wave & 3;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int KB = g.K / 128;
  const int kb0 = split * KB / g.splits, kb1 = (split + 1) * KB / g.splits;
  const int nb = kb1 - kb0;
  uint8_t* Xl = lds;
  uint8_t* Wl = lds + XS * XB;
  uint8_t* Sl = Wl + WS * WBYTES;
  const uint32_t xbase = lds_off(Xl), wbase = lds_off(Wl), sbase = lds_off(Sl);

  // ---- direct loads: wave-uniform base (SGPRs) + per-lane byte offset.
  // Activations: load p covers rows 32 p + 4 wave + (lane >> 4) (waves
  // 0-3 take one more load when TM is odd), slot (lane & 15) of a row
  // holding chunk slot ^ (row & 15); rows past M (last load only) reload row
  // M-1, never stored.  Codes: subtiles 2 wave, 2 wave + 1 of 16 (past N: the
  // last one).  Chunk `wave` of the 8 scale / min chunks: the scales (even)
  // or mins (odd) of group wave >> 1.
  const int r0 = 4 * wave + (lane >> 4);
  const int cx = (lane & 15) ^ xswz(r0 & 15);
  const uint32_t xoff = (uint32_t)(r0 * g.lda + 8 * cx) * 2u;
  const uint32_t xoff_last =
      (uint32_t)((min(32 * (NX - 1) + r0, g.M - 1) - 32 * (NX - 1)) * g.lda + 8 * cx) * 2u;
  const uint32_t coff = (uint32_t)lane * 16u, soff = (uint32_t)lane * 4u;
  const int gi = min(nt * 4 + (wave >> 1), g.N / 64 - 1);
  const _Float16* sbase_g = ((wave & 1) ? g.minv : g.scale) + (int64_t)gi * g.K;
  auto blk = [&](int i) __attribute__((always_inline)) { return kb0 + min(i, nb - 1); };
  auto issue_x = [&](int i) __attribute__((always_inline)) {
    const int kb = blk(i);
    const uint32_t base = xbase + (i & 1) * XB + wave * 1024;
    unr<NX>([&](auto p_) {
      constexpr int p = decltype(p_)::value;
      dma16s(g.A + (int64_t)(32 * p) * g.lda + kb * 128, p == NX - 1 ? xoff_last : xoff,
             __builtin_amdgcn_readfirstlane(base + p * 8192));
    });
  };
  auto issue_ws = [&](int i) __attribute__((always_inline)) {
    const int kb = blk(i);
    const uint32_t wb = wbase + (i & 3) * WBYTES + 2 * wave * 1024;
    unr<2>([&](auto h_) {
      constexpr int h = decltype(h_)::value;
      const int n16 = min(nt * 16 + 2 * wave + h, g.N / 16 - 1);
      dma16s(g.B + ((int64_t)n16 * KB + kb) * 1024, coff,
             __builtin_amdgcn_readfirstlane(wb + h * 1024));
    });
    dma4s(sbase_g + kb * 128, soff,
          __builtin_amdgcn_readfirstlane(sbase + (i & 3) * SBYTES + wave * SCH));
  };

  const DqConst dq{0x000F000Fu, 0x00F000F0u, in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
  f32x4 acc[TM][4];
  unr<TM>([&](auto i_) {
    unr<4>([&](auto t_) { acc[decltype(i_)::value][decltype(t_)::value] = f32x4{0.f, 0.f, 0.f, 0.f}; });
  });
  f16x8 x[TM], w[4];
  uint32_t c0[4], c1[4];  // codes of the wave's first / second step of a block
  uint32_t sd;            // this lane's scale-or-min dword of the block
  // k-step j of a k-block: lane quarter kq covers k = 32 kq + 8 j .. +7
  auto read_x = [&](f16x8& o, int xs, auto j_, int i) __attribute__((always_inline)) {
    constexpr int j = decltype(j_)::value;
    o = *(const f16x8*)(Xl + xs * XB + (16 * i + r16) * 256 + 16 * ((4 * kq + j) ^ xswz(r16)));
  };
  // Codes: dwords J0, J0 + 1 of the lane's 16 bytes.  Scales: the lane
  // quarter's 16 k (32 kq + 8 J0 ..) need 8 scale and 8 min dwords; lane d
  // of the quarter's row of 16 holds scale dword d (d < 8) or min dword d - 8.
  const int sd_off = (2 * wcol + (r16 >> 3)) * SCH + 64 * kq + 32 * PH + 4 * (r16 & 7);
  auto read_cs = [&](int wsg) __attribute__((always_inline)) {
    const uint8_t* cp = Wl + wsg * WBYTES + 4 * wcol * 1024 + lane * 16 + 8 * PH;
    unr<4>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      const u32x2 v = *(const u32x2*)(cp + t * 1024);
      c0[t] = v[0];
      c1[t] = v[1];
    });
    sd = *(const uint32_t*)(Sl + wsg * SBYTES + sd_off);
  };
  // expansion of the wave's step s (0: first, 1: second) of the block
  auto expand = [&](const uint32_t (&c)[4], auto s_) __attribute__((always_inline)) {
    constexpr int s = decltype(s_)::value;
    const u32x4 sv = {row_bcast<4 * s + 0>(sd), row_bcast<4 * s + 1>(sd), row_bcast<4 * s + 2>(sd),
                      row_bcast<4 * s + 3>(sd)};
    const u32x4 mv = {row_bcast<8 + 4 * s + 0>(sd), row_bcast<8 + 4 * s + 1>(sd),
                      row_bcast<8 + 4 * s + 2>(sd), row_bcast<8 + 4 * s + 3>(sd)};
    unr<4>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      w[t] = dequant8(c[t], sv, mv, dq);
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using JA = std::integral_constant<int, J0>;      // first step of a block
  using JB = std::integral_constant<int, J0 + 1>;  // second step

  // One step: MFMAs with the held operands, next step's activations from
  // buffer xs at k-step jn, and the next step's weights from codes `cn`
  // (step sn).  `NR` LDS reads (codes and scales of the next block, issued
  // just before) come first in the issue order.
  auto step = [&](int xs, auto jn_, const uint32_t (&cn)[4], auto sn_, auto nr_)
      __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_)::value;
    constexpr int T0 = NR == 0 ? 0 : (TM >= 4 ? 2 : (TM >= 2 ? 1 : 0));
    constexpr int VPM = (60 + 4 * (TM - T0) - 1) / (4 * (TM - T0));
    const f16x8 wc[4] = {w[0], w[1], w[2], w[3]};
    unr<TM>([&](auto i_) {
      constexpr int r = decltype(i_)::value;
      const f16x8 xr = x[r];
      unr<4>([&](auto t_) {
        constexpr int t = decltype(t_)::value;
        acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc[t], xr, acc[r][t], 0, 0, 0);
      });
      read_x(x[r], xs, jn_, r);
    });
    expand(cn, sn_);
    unr<NR>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
    unr<TM>([&](auto i_) {
      constexpr int r = decltype(i_)::value;
      unr<4>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (r >= T0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      });
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: weights of blocks 0..2, activations of blocks 0 and 1
  issue_ws(0);
  issue_x(0);
  issue_ws(1);
  issue_x(1);
  issue_ws(2);
  wait_vm<2 * NWS + NX>();  // block 0's loads (own)
  __builtin_amdgcn_s_barrier();
  unr<TM>([&](auto i_) { read_x(x[decltype(i_)::value], 0, JA(), decltype(i_)::value); });
  read_cs(0);
  expand(c0, I0());
  __builtin_amdgcn_sched_barrier(0);

  for (int i = 0; i < nb; ++i) {
    // first step of block i; next: the second step (codes already held)
    step(i & 1, JB(), c1, I1(), I0());
    // block boundary: this wave's activations of block i are in registers
    wait_vm<NWS, 0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_x(i + 2);
    issue_ws(i + 3);
    __builtin_amdgcn_sched_barrier(0);
    // second step of block i; next: the first step of block i+1
    read_cs((i + 1) & 3);
    step((i + 1) & 1, JA(), c0, I0(), std::integral_constant<int, 5>());
  }
  wait_vm<0, 0>();  // every direct load and LDS read of this wave is done
  __builtin_amdgcn_s_barrier();

  // ---- add the two halves: the PH = 0 wave finalises row tiles [0, H), the
  // PH = 1 wave [H, TM); each writes the other's half of its sums to LDS
  constexpr int H = (TM + 1) / 2;
  float* xch = (float*)lds + wcol * (TM * 4 * 4 * 64);  // [tile][t][e][lane]
  unr<TM>([&](auto i_) {
    constexpr int i = decltype(i_)::value;
    if constexpr ((PH == 0) == (i >= H)) {
      unr<4>([&](auto t_) {
        constexpr int t = decltype(t_)::value;
        *(f32x4*)(xch + ((i * 4 + t) * 64 + lane) * 4) = acc[i][t];
      });
    }
  });
  wait_vm<0, 0>();  // the exchange writes are done before the barrier
  __builtin_amdgcn_s_barrier();
  const int n_wave = nt * 256 + wcol * 64;
  if (n_wave >= g.N) return;
  unr<TM>([&](auto i_) {
    constexpr int i = decltype(i_)::value;
    if constexpr ((PH == 0) == (i < H)) {
      const int m = 16 * i + r16;
      unr<4>([&](auto t_) {
        constexpr int t = decltype(t_)::value;
        const int n = n_wave + 16 * t + 4 * kq;
        f32x4 v = acc[i][t] + *(const f32x4*)(xch + ((i * 4 + t) * 64 + lane) * 4);
        if (m >= g.M) return;
        if (g.P) {
          // tile-major partials: one store instruction writes 1 KB contiguous
          const int64_t pi =
              ((((int64_t)split * g.ntiles + nt) * 4 + wcol) * TM + i) * 4 + t;
          *(f32x4*)(g.P + (pi * 64 + lane) * 4) = v;
          return;
        }
        if (g.relu) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.0f);
        }
        if (g.res) {
          const f16x4 rr = *(const f16x4*)(g.res + m * g.ldr + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += (float)rr[e];
        }
        f16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (_Float16)v[e];
        *(f16x4*)(g.Y + m * g.ldy + n) = o;
      });
    }
  });
}

template <int TM>
__global__ __launch_bounds__(512, 1) void k_gemm_dq(DqArgs g) {
  constexpr int BYTES = XS * 16 * TM * 256 + WS * (WBYTES + SBYTES);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[BYTES];
  static_assert(4 * TM * 4 * 4 * 64 * 4 <= BYTES, "the exchange fits in LDS");
  // workgroups on one XCD (id % 8) take a contiguous run of (split, column
  // tile) pairs, split-major, so they share activation k-slices in L2
  const int total = g.ntiles * g.splits;
  int id = blockIdx.x;
  const int per_xcd = total / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  const int split = id / g.ntiles, nt = id % g.ntiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4)
    dq_pair<TM, 0>(g, lds, wave, nt, split);
  else
    dq_pair<TM, 1>(g, lds, wave, nt, split);
}

// Sums the split partials of k_gemm_dq in split order and applies the
// epilogue.  Partial layout: [split][column tile][column group][row tile]
// [subtile][lane] f32x4, lane l holding row 16 (row tile) + l % 16 and
// columns 16 (subtile) + 4 (l / 16) .. +3 of its group; one thread per f32x4
// of a split, so the partial reads are contiguous.  The split count is a
// template argument: a thread issues the loads of all S splits before the
// first add (a run-time loop waits for each load in turn), and the adds
// still go in split order.
template <int S>
__global__ __launch_bounds__(256) void k_dq_reduce(const float* __restrict__ P, int ntiles, int tm,
                                                   int M, int N, const _Float16* __restrict__ res,
                                                   int64_t ldr, int relu, _Float16* __restrict__ Y,
                                                   int64_t ldy) {
  const int64_t per_split = (int64_t)ntiles * 4 * tm * 4 * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < per_split; q += stride) {
    const int lane = (int)(q & 63), t = (int)((q >> 6) & 3);
    int64_t rest = q >> 8;
    const int i = (int)(rest % tm);
    rest /= tm;
    const int wcol = (int)(rest & 3), nt = (int)(rest >> 2);
    const int m = 16 * i + (lane & 15);
    const int n = nt * 256 + wcol * 64 + 16 * t + 4 * (lane >> 4);
    if (m >= M || n >= N) continue;
    f32x4 p[S];
#pragma unroll
    for (int s = 0; s < S; ++s) p[s] = __builtin_nontemporal_load((const f32x4*)(P + (s * per_split + q) * 4));
    f32x4 v = p[0];
#pragma unroll
    for (int s = 1; s < S; ++s) v += p[s];
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

template <int N = 2, class F>
bool with_splits(int n, F&& f) {
  if constexpr (N > 16) {
    (void)n;
    (void)f;
    return false;
  } else {
    if (n == N) {
      f(std::integral_constant<int, N>());
      return true;
    }
    return with_splits<N + 1>(n, f);
  }
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
  {
    Prof prof("gemm_q4_skinny", st);  // the product alone; the reduce is timed on its own
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, a); };
    switch (T) {
      case 1: go(k_gemm_dq<1>); break;
      case 2: go(k_gemm_dq<2>); break;
      case 3: go(k_gemm_dq<3>); break;
      case 4: go(k_gemm_dq<4>); break;
      case 5: go(k_gemm_dq<5>); break;
      case 6: go(k_gemm_dq<6>); break;
      case 7: go(k_gemm_dq<7>); break;
      case 8: go(k_gemm_dq<8>); break;
      default: go(k_gemm_dq<9>); break;
    }
  }
  hp_status s = launch_ok("k_gemm_dq");
  if (s != HP_OK || splits == 1) return s;
  const int64_t per_split = (int64_t)a.ntiles * 4 * T * 4 * 64;
  const int blocks = (int)std::min<int64_t>(cdiv(per_split, 256), 8192);
  Prof prof_r("gemm_splitk_reduce", st);
  const bool known = with_splits(splits, [&](auto s_) {
    hipLaunchKernelGGL(k_dq_reduce<decltype(s_)::value>, dim3(blocks), dim3(256), 0, st,
                       (const float*)partials, a.ntiles, T, (int)M, w.n, (const _Float16*)res, ldr,
                       a.relu, (_Float16*)y, ldy);
  });
  if (!known) return fail(HP_ERR_SHAPE, "split count %d outside 2..16", splits);
  return launch_ok("k_dq_reduce");
}

}  // namespace hp
