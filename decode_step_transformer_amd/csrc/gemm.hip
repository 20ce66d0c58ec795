// Dequant-fused MFMA matrix product y = act(x·w) + res for the FlexGen layer
// ([FlexGen] paper notes, background section: Q/K/V/O projections and the
// two MLP products are all x·w; section 5: int4 weights are converted back
// to FP16 before the product).
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//  * A workgroup is 8 waves and owns a BM x 128 output tile (BM = all M
//    rows, 16 TM); wave w owns the 16 output columns [16 w, 16 w + 16) for
//    all BM rows.  The product is bound by streaming the fp16 weights, so
//    each wave keeps three k-blocks of its weight fragments in flight in
//    registers (48 VGPRs) and a CU holds up to 16 waves.
//  * The activation tile x[BM][128] of each k-block is staged through LDS
//    (three stages, rows padded by 16 B) and shared by the 8 waves.
//  * Weight fragments go straight from HBM to registers, four 16-byte chunks
//    per lane and subtile per k-block.  The fp16 weight layout is fragment-
//    major (k-step j of a block is k = 32 j .. 32 j + 31, lane quarter q
//    holding 32 j + 8 q .. + 7, and the 64 lanes' fragments are contiguous),
//    so each load instruction reads one contiguous 1 KB, and the tiles of
//    one k-block are adjacent, so the workgroups of a split, which move
//    through k together, read one contiguous window of memory at a time.
//    With rows of w^T (16 rows x 64 bytes per instruction, rows a power of
//    two apart) the products ran 8-21% slower; with each column tile's
//    k-blocks adjacent instead (2048 separate streams) 8-11% slower.
//  * MFMA operand A is the weight fragment (16 output columns), operand B the
//    activation fragment (16 rows), so each lane ends with 4 consecutive
//    output columns of one row: 8-byte stores.
//  * Skinny products (M <= 144, the decode step) split k over workgroups;
//    partial sums go to fp32 scratch and a second kernel adds them in split
//    order, so the result depends only on (k, n), never on M.  Skinny int4
//    products run on the 8-wave kernel of gemm_dec.hip (same split rule);
//    tall ones expand int4 weights to fp16 and run k_gemm16.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "dequant_dev.h"

namespace hp {

constexpr int BK = 128;        // k-block (one packed q4 tile in depth)
constexpr int LDS_ROW = 136;   // halves per staged activation row (128 + 8 pad)
constexpr int SKINNY_M = (int)kSkinnyM;  // largest M handled as one row tile with split-k


// Calls f(integral_constant<0>) .. f(integral_constant<N-1>): compile-time
// indices, so register arrays indexed inside f stay in registers.
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (N > 0) {
    unroll<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

struct GemmArgs {
  const _Float16* A;
  int64_t lda, M;
  const _Float16* B;  // fragment-major fp16 tiles (the HP_F16 layout)
  int K, N, splits, mtiles;  // split s covers k-blocks [s KB / splits, (s+1) KB / splits)
  const _Float16* res;
  int64_t ldr;
  int relu;
  _Float16* Y;
  int64_t ldy;
  float* P;  // split partials [split][M][N] or null
};

constexpr int NS = 3;  // LDS activation stages and weight register slots

constexpr int F_WAVES = 8;                 // waves per workgroup
constexpr int F_COLS = 16 * F_WAVES;       // output columns per workgroup

// Workgroup tile order: workgroups on the same XCD (id % 8) take a contiguous
// run of tiles, and runs sweep 4 row tiles at a time so that concurrently
// running tiles share activation and weight k-slices in L2.
__device__ __forceinline__ void tile_of(const GemmArgs& g, int& mt, int& nt) {
  const int ntiles = (g.N + F_COLS - 1) / F_COLS;
  const int total = g.mtiles * ntiles;
  int id = blockIdx.x;
  const int per_xcd = total / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  constexpr int GM = 4;
  const int group = id / (GM * ntiles);
  const int first_m = group * GM;
  const int gm = min(GM, g.mtiles - first_m);
  mt = first_m + (id % (GM * ntiles)) % gm;
  nt = (id % (GM * ntiles)) / gm;
}

// One wave's part of a workgroup tile: TM 16-row tiles starting at row tile
// rt0 of the workgroup's rows (from m0), times the 16 output columns of wave
// column wcol.  All NT threads of the workgroup stage SR activation rows per
// k-block into As (NS stages of SR x LDS_ROW halves).
template <int TM, int NT, int SR>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, _Float16* As_, int tid, int wcol,
                                          int rt0, int64_t m0, int nt) {
  const int lane = tid & 63;
  const int KB = g.K / BK;
  auto As = [&](int stage) __attribute__((always_inline)) { return As_ + stage * (SR * LDS_ROW); };
  const int n_wave = nt * F_COLS + wcol * 16;
  const bool wave_on = n_wave < g.N;
  // a wave past the last column reloads the last subtile (never stored), so
  // every load is unconditional
  const int n_ld = min(n_wave, g.N - 16);
  const int split = blockIdx.y;
  const int kb0 = split * KB / g.splits, kb1 = (split + 1) * KB / g.splits;
  auto clampk = [&](int kb) __attribute__((always_inline)) { return min(kb, kb1 - 1); };

  // ---- activation tile loader: CH 16-byte chunks per thread.  Rows past M
  // reload row M-1 (their outputs are never stored).
  constexpr int CH = SR * 16 / NT;
  static_assert(CH * NT == SR * 16, "staged rows must split evenly over the threads");
  u32x4 areg[CH];
  // chunk c of this thread: row (tid >> 4) + (NT / 16) c, column (tid & 15) * 8
  const _Float16* abase = g.A + (int64_t)((tid & 15) * 8);
  const int64_t arow0 = m0 + (tid >> 4);
  auto load_a = [&](int kb) __attribute__((always_inline)) {
    unroll<CH>([&](auto c_) {
      constexpr int c = decltype(c_)::value;
      const int64_t m = min(arow0 + (NT / 16) * c, g.M - 1);
      areg[c] = *(const u32x4*)(abase + m * g.lda + (int64_t)kb * BK);
    });
  };
  auto store_a = [&](int stage) __attribute__((always_inline)) {
    unroll<CH>([&](auto c_) {
      constexpr int c = decltype(c_)::value;
      const int chunk = tid + NT * c;
      *(u32x4*)(As(stage) + (chunk >> 4) * LDS_ROW + (chunk & 15) * 8) = areg[c];
    });
  };

  // ---- weight fragments ----
  const int kq = lane >> 4, r16 = lane & 15;
  struct Raw {
    u32x4 c[4];  // the 4 k-steps of one k-block
  };
  // fragment-major weight tiles (4 KB per 16 columns x 128 inputs, the tiles
  // of one k-block adjacent): k-step j of block kb is one contiguous 1 KB,
  // lane L's 16 bytes at L * 16
  const _Float16* Bh = g.B + ((int64_t)(n_ld / 16) * 256 + lane) * 8;
  const int64_t kb_stride = (int64_t)(g.N / 16) * 2048;  // halves per k-block of tiles
  auto load_b = [&](Raw& R, int kb) __attribute__((always_inline)) {
    const u32x4* p = (const u32x4*)(Bh + (int64_t)kb * kb_stride);
    unroll<4>([&](auto j_) {
      constexpr int j = decltype(j_)::value;
      R.c[j] = p[64 * j];
    });
  };

  f32x4 acc[TM];
  unroll<TM>([&](auto i_) { acc[decltype(i_)::value] = f32x4{0.f, 0.f, 0.f, 0.f}; });

  // ---- one MFMA k-step (32 deep): fragments of (stage, j) ----
  f16x8 xa[TM], xb[TM], wa, wb;
  auto read_x = [&](f16x8 (&x)[TM], int stage, int j) __attribute__((always_inline)) {
    const _Float16* Ab = As(stage) + (16 * rt0 + r16) * LDS_ROW + 8 * kq + 32 * j;
    unroll<TM>([&](auto i_) {
      constexpr int i = decltype(i_)::value;
      x[i] = *(const f16x8*)(Ab + 16 * i * LDS_ROW);
    });
  };
  auto make_w = [&](f16x8& w, const Raw& R, auto j_) __attribute__((always_inline)) {
    w = as_f16x8(R.c[decltype(j_)::value]);
  };
  auto mma = [&](const f16x8& w, const f16x8 (&x)[TM]) __attribute__((always_inline)) {
    unroll<TM>([&](auto i_) {
      constexpr int i = decltype(i_)::value;
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w, x[i], acc[i], 0, 0, 0);
    });
  };
  // issue order inside one k-step: the LDS reads of the next step first,
  // then the MFMAs
  auto interleave = [&]() __attribute__((always_inline)) {
    unroll<TM>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
    unroll<TM>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); });
  };

  Raw r0, r1, r2;
  // prologue: stages 0 and 1 hold activation blocks kb0 and kb0+1; weight
  // slots 0 and 1 hold kb0 and kb0+1; registers hold block kb0+2
  load_a(kb0);
  load_b(r0, kb0);
  store_a(0);
  load_a(clampk(kb0 + 1));
  store_a(1);
  load_a(clampk(kb0 + 2));
  // issued after the last activation load, so that on entry to the loop the
  // activation registers are followed by one k-block of weight loads, as at
  // every back edge: the compiler's memory-counter wait at the loop head is
  // then the steady-state one instead of a wait for the next weights too
  load_b(r1, clampk(kb0 + 1));
  __syncthreads();
  read_x(xa, 0, 0);
  make_w(wa, r0, std::integral_constant<int, 0>());

  // k-block kb in stage st % 3, weights in `cur`; `nxt` holds kb+1, `fill`
  // receives kb+2.  At entry xa/wa hold the fragments of (kb, j = 0).
  auto step = [&](const Raw& cur, const Raw& nxt, Raw& fill, int kb) __attribute__((always_inline)) {
    const int st = (kb - kb0) % NS, st1 = (kb - kb0 + 1) % NS, st2 = (kb - kb0 + 2) % NS;
    __syncthreads();  // every wave is done with stage st2 (block kb-1)
    store_a(st2);
    load_a(clampk(kb + 3));
    load_b(fill, clampk(kb + 2));
    __builtin_amdgcn_sched_barrier(0);
    read_x(xb, st, 1);
    mma(wa, xa);
    make_w(wb, cur, std::integral_constant<int, 1>());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_x(xa, st, 2);
    mma(wb, xb);
    make_w(wa, cur, std::integral_constant<int, 2>());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_x(xb, st, 3);
    mma(wa, xa);
    make_w(wb, cur, std::integral_constant<int, 3>());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_x(xa, st1, 0);
    mma(wb, xb);
    make_w(wa, nxt, std::integral_constant<int, 0>());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  // whole rounds of 3 steps, then the remainder: no branch inside the loop
  // body, so the accumulators never pass through a join
  int kb = kb0;
  for (; kb + 3 <= kb1; kb += 3) {
    step(r0, r1, r2, kb);
    step(r1, r2, r0, kb + 1);
    step(r2, r0, r1, kb + 2);
  }
  if (kb < kb1) step(r0, r1, r2, kb);
  if (kb + 1 < kb1) step(r1, r2, r0, kb + 1);

  if (!wave_on) return;
  // ---- epilogue: lane holds rows m = m0 + 16 i + r16, columns n .. n+3 ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + 16 * (rt0 + i) + r16;
    if (m >= g.M) continue;
    const int n = n_wave + 4 * kq;
    f32x4 v = acc[i];
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

// Products with one row tile per workgroup (or any M): 8 waves, each with all
// TM row tiles of its 16 columns; the staged rows are padded to a multiple
// of 32 so that the 512 threads split them evenly.
template <int TM>
__global__ __launch_bounds__(512, 2) void k_gemm(GemmArgs g) {
  constexpr int SR = 32 * ((TM + 1) / 2);
  __shared__ __attribute__((aligned(16))) _Float16 As[NS * SR * LDS_ROW];
  int mt, nt;
  tile_of(g, mt, nt);
  const int wave = threadIdx.x >> 6;
  gemm_tile<TM, 512, SR>(g, As, threadIdx.x, wave, 0, (int64_t)mt * 16 * TM, nt);
}

// Calls f(std::integral_constant<int, n>()) for a split count n in [2, 16]
// (the range split_for produces) and returns true; false otherwise.
template <int N = 2, class F>
static bool with_split_count(int n, F&& f) {
  if constexpr (N > 16) {
    (void)n;
    (void)f;
    return false;
  } else {
    if (n == N) {
      f(std::integral_constant<int, N>());
      return true;
    }
    return with_split_count<N + 1>(n, f);
  }
}

// Sums split-k partials in split order, then applies the epilogue.  The
// split count is a template argument so that a thread issues the loads of
// all S splits before the first add (with a run-time count each load waited
// for the previous add; the partials of an M = 64 product are a few MB, so
// the sum is bound by that latency); the adds still go in split order.
template <int S>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ P, int64_t M,
                                                       int N, const _Float16* __restrict__ res,
                                                       int64_t ldr, int relu,
                                                       _Float16* __restrict__ Y, int64_t ldy) {
  const int64_t quads = M * (N / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const int64_t m = q / (N / 4);
    const int n = (int)(q % (N / 4)) * 4;
    f32x4 p[S];
#pragma unroll
    for (int s = 0; s < S; ++s) p[s] = *(const f32x4*)(P + ((int64_t)s * M + m) * N + n);
    f16x4 r = {};
    if (res) r = *(const f16x4*)(res + m * ldr + n);
    f32x4 v = p[0];
#pragma unroll
    for (int s = 1; s < S; ++s) v += p[s];
    if (relu) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.0f);
    }
    if (res) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += (float)r[e];
    }
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (_Float16)v[e];
    *(f16x4*)(Y + m * ldy + n) = o;
  }
}

// Split factors for skinny products: functions of (k, n) only, so a row's
// result never depends on how many rows the product has.
//
// 8-wave int4 kernel (one workgroup per CU): minimise, in units of one
// k-block's time, rounds * k-blocks per split + the split partials' traffic
// (about 2.4e-4 k-block times per output column and split).
static int split_rs(int32_t k, int32_t n) {
  const int KB = k / BK;
  const int64_t ntiles = cdiv(n, 256);
  const double pc = 2.43e-4 * n;
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= KB && s <= 16; ++s) {
    const double cost = (double)cdiv(ntiles * s, 256) * (double)cdiv(KB, s) + (s > 1 ? s * pc : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}
// 8-wave fp16 kernel: at least 192 workgroups where the k-blocks allow (each
// keeps up to 96 KB of weight fragments in flight; at the 6.7B QKV shape 2
// splits over 96 column tiles ran 26.0 + 6.3 us against 28.0 + 6.4 for 4).
static int split_for(int32_t k, int32_t n) {
  const int KB = k / BK;
  const int ntiles = (int)cdiv(n, F_COLS);
  const int want = (int)cdiv(192, ntiles);
  for (int d = 1; d <= KB && d <= 16; ++d)
    if (KB % d == 0 && d >= want) return d;
  int best = 1;
  for (int d = 1; d <= KB && d <= 16; ++d)
    if (KB % d == 0) best = d;
  return best;
}

size_t gemm_ws_bytes(int64_t M, int32_t k, int32_t n, int32_t fmt) {
  if (M <= 0) return 0;
  if (M > SKINNY_M) return fmt == HP_Q4 ? (size_t)pad_ld(k) * (size_t)n * 2 : 0;  // fp16 expansion
  if (fmt == HP_Q4) {  // tile-major partials of k_gemm_dq: padded to 256 columns, 16-row tiles
    const int s = split_rs(k, n);
    return s > 1 ? (size_t)s * (size_t)cdiv(n, 256) * 256 * (size_t)cdiv(M, 16) * 16 * sizeof(float)
                 : 0;
  }
  const int s = split_for(k, n);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)n * sizeof(float) : 0;
}

// ------------------------------------------------ allocation-free scratch
// Split-k partial sums for hp_gemm_noalloc: a fixed array in the code
// object, one copy per GPU, resident until the process ends.  In host code
// `scratch` names a host-side stand-in, never a device address: kernels get
// the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[64];

hp_status static_scratch(void** ptr) {
  int dev = -1;
  hp_status s = hip_ok(hipGetDevice(&dev), "hipGetDevice");
  if (s != HP_OK) return s;
  if (dev < 0 || dev >= 64) return fail(HP_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if ((s = hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress")) != HP_OK)
      return s;
    if (!p) return fail(HP_ERR_HIP, "hipGetSymbolAddress returned NULL");
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return HP_OK;
}

template <int TM>
static void launch_tm(const GemmArgs& a, dim3 grid, hipStream_t st) {
  Prof prof("gemm_f16_skinny", st);
  hipLaunchKernelGGL(k_gemm<TM>, grid, dim3(512), 0, st, a);
}

hp_status launch_gemm(const void* x, int64_t ldx, const hp_mat& w, int64_t M, const void* res,
                      int64_t ldr, bool relu, void* y, int64_t ldy, void* ws, hipStream_t st) {
  if (M == 0) return HP_OK;
  const bool q4 = w.fmt == HP_Q4;
  if (M <= SKINNY_M) {
    const int splits = q4 ? split_rs(w.k, w.n) : split_for(w.k, w.n);
    // int4: the kernel and its split-k reduce (tile-major partials) in gemm_dec.hip
    if (q4) return launch_gemm_dq(x, ldx, w, M, res, ldr, relu, y, ldy, splits, (float*)ws, st);
    GemmArgs a;
    a.A = (const _Float16*)x;
    a.lda = ldx;
    a.M = M;
    a.B = (const _Float16*)w.data;
    a.K = w.k;
    a.N = w.n;
    a.res = (const _Float16*)res;
    a.ldr = ldr;
    a.relu = relu ? 1 : 0;
    a.Y = (_Float16*)y;
    a.ldy = ldy;
    a.splits = splits;
    a.mtiles = 1;
    a.P = splits > 1 ? (float*)ws : nullptr;
    const dim3 grid((unsigned)cdiv(w.n, F_COLS), splits);
    switch ((int)cdiv(M, 16)) {
      case 1: launch_tm<1>(a, grid, st); break;
      case 2: launch_tm<2>(a, grid, st); break;
      case 3: launch_tm<3>(a, grid, st); break;
      case 4: launch_tm<4>(a, grid, st); break;
      case 5: launch_tm<5>(a, grid, st); break;
      case 6: launch_tm<6>(a, grid, st); break;
      case 7: launch_tm<7>(a, grid, st); break;
      case 8: launch_tm<8>(a, grid, st); break;
      default: launch_tm<9>(a, grid, st); break;
    }
    hp_status s = launch_ok("k_gemm");
    if (s != HP_OK || splits == 1) return s;
    const int64_t quads = M * (w.n / 4);
    const int blocks = (int)std::min<int64_t>(cdiv(quads, 256), 8192);
    Prof prof("gemm_splitk_reduce", st);
    const bool known = with_split_count(splits, [&](auto s_) {
      hipLaunchKernelGGL(k_splitk_reduce<decltype(s_)::value>, dim3(blocks), dim3(256), 0, st,
                         (const float*)ws, M, w.n, (const _Float16*)res, ldr, relu ? 1 : 0,
                         (_Float16*)y, ldy);
    });
    if (!known) return fail(HP_ERR_SHAPE, "k_splitk_reduce: split count out of range");
    return launch_ok("k_splitk_reduce");
  }
  // tall products: fp16 MFMA kernel over LDS tiles; int4 weights are first
  // expanded to fp16 into the scratch buffer
  if (q4) {
    hp_status s = launch_expand_q4(w, ws, pad_ld(w.k), st);
    if (s != HP_OK) return s;
    return launch_gemm16(x, ldx, ws, pad_ld(w.k), w.k, w.n, M, res, ldr, relu, y, ldy, st);
  }
  return launch_gemm16(x, ldx, w.data, 0, w.k, w.n, M, res, ldr, relu, y, ldy, st);
}

}  // namespace hp
