// Top-K sparse attention over the KV cache ([FlexGen] paper notes, section 5,
// sparse attention): for the decode query of a (request, head), the scores
// against every cached key are formed, the indices of the K largest are
// found, the other tokens are dropped, and only the V rows at those indices
// are read; the output is the attention over the kept rows.  With K = 10% of
// the rows, a step reads the whole K cache but a tenth of the V cache.
//
// One wave per (request, head), three passes:
//  1. K is streamed in chunks of 4 loads (two register sets, one chunk in
//     flight while the other is scored); the scores of all T rows go to LDS.
//  2. Exact selection: every lane holds the scores of rows lane, lane + 64,
//     ... as order-preserving 32-bit keys; a threshold is built bit by bit
//     from the top (keep a bit if at least K keys reach the candidate; stop
//     as soon as exactly K do, else after 32 rounds at the K-th largest key).
//     Rows above it are kept, and rows equal to it by ascending index until
//     K are kept (ties go to the lower index); ballot prefix counts give every
//     kept row its place in an ascending list in LDS.
//  3. The kept V rows are gathered (two register sets in flight) and summed
//     with weights exp(z - max); the maximum is the top score, known before
//     the pass, so no rescaling is needed.
// Paged caches (PAGED): the request's page numbers (up to 64) sit one per
// lane; a K load's rows lie in one page (RPI rows from a multiple of RPI,
// RPI | 64 | page rows), read with v_readlane, and every gathered V row looks
// up its own page (a lane shuffle, or the table in memory past 64 pages).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "decode_dev.h"
#include "dequant_dev.h"

namespace hp {

struct TopkArgs {
  const _Float16* qkv;  // [b][3 h1]: the query in columns [0, h1)
  int h1, H, pos;       // visible rows [0, pos + step + 1)
  const int32_t* dpos;  // step added to pos (device int32), or null
  int topk;             // kept rows (at most T); 0: ceil(T / 10)
  int cap;
  const void* k;
  const void* v;
  const uint32_t* ksm;
  const uint32_t* vsm;
  _Float16* out;  // [b][h1]
  int32_t* idx;   // [b][H][K] kept rows in ascending order, or null
  const int32_t* rpos;   // each request's own row of its new token (at most pos), or null
  const int32_t* pages;  // page table [b][cap / PR] of a paged cache (PAGED)
  int PR, pool;
};

// Order-preserving key of a score: a larger score gives a larger key; -0 and
// +0 give the same key (s + 0 turns -0 into +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave-uniform sum of a small integer: DPP within each row of 16 lanes, then
// the four rows' sums read as scalars.
__device__ __forceinline__ int wave_total(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, DPP_XOR1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_XOR2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_HALF_MIRROR, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_MIRROR, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// This lane's 16-byte slices (and scale/min pairs) of the cache rows row[u]:
// rel[u] is the cache row of logical row row[u], less row[u] (the request's
// first row for a contiguous cache).
template <int D, bool Q4, int U>
__device__ __forceinline__ void load_rows(DecPart<U, Q4>& X, const uint8_t* cache, const uint8_t* smc,
                                          const int64_t (&rel)[U], const int (&row)[U],
                                          uint32_t lane_off, uint32_t lane_soff) {
  using S = DecShape<D, Q4>;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint8_t* cb = cache + rel[u] * S::RB;
    X.c[u] = __builtin_nontemporal_load((const u32x4*)(cb + ((uint32_t)row[u] * S::RB + lane_off)));
    if constexpr (Q4) {
      const uint8_t* sb = smc + rel[u] * (4 * S::G);
      X.sm[u] = *(const uint32_t*)(sb + ((uint32_t)row[u] * (4 * S::G) + lane_soff));
    }
  }
  asm volatile("" ::: "memory");  // keeps each prefetch where it is issued
}

// NS: score slots per lane (T <= 64 NS)
template <int D, bool Q4, int NS, bool PAGED>
__global__ __launch_bounds__(64) void k_topk_attn(TopkArgs a) {
  using S = DecShape<D, Q4>;
  constexpr int LPR = S::LPR, RPI = S::RPI, RB = S::RB, G = S::G;
  constexpr int UK = 4, CRK = UK * RPI;  // rows per K chunk
  constexpr int UV = 2, CRV = UV * RPI;  // rows per V chunk
  __shared__ float sc[64 * NS];          // scores of rows [0, T)
  __shared__ int sel[64 * NS];           // kept rows, ascending

  const int lane = threadIdx.x;
  const int qd = lane % LPR, rho = lane / LPR;
  const int h = blockIdx.x % a.H, r = blockIdx.x / a.H;
  const int T = a.rpos ? min(max(a.rpos[r], 0), a.pos) + 1 : a.pos + (a.dpos ? *a.dpos : 0) + 1;
  const int K = a.topk > 0 ? min(a.topk, T) : (T + 9) / 10;
  const int64_t rowbase = ((int64_t)r * a.H + h) * a.cap;
  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  const uint8_t* ksb = (const uint8_t*)a.ksm;
  const uint8_t* vsb = (const uint8_t*)a.vsm;
  const int prs = PAGED ? __builtin_ctz(a.PR) : 0;  // page rows are a power of two
  const int npg = PAGED ? a.cap >> prs : 0;
  int pg_lane = 0;
  if constexpr (PAGED) {
    if (npg <= 64 && lane < npg) pg_lane = min(max(a.pages[(int64_t)r * npg + lane], 0), a.pool - 1);
  }
  // cache row of logical row j, less j: j wave-uniform (a K load), or per lane
  // (a gathered V row)
  // (page's first row) - (page slot of j) x (page rows)
  auto page_row = [&](int pg, int j) __attribute__((always_inline)) -> int64_t {
    return ((int64_t)pg * a.H + h - (j >> prs)) * a.PR;
  };
  auto table = [&](int j) __attribute__((always_inline)) {
    return min(max(a.pages[(int64_t)r * npg + (j >> prs)], 0), a.pool - 1);
  };
  auto rel_uniform = [&](int j) __attribute__((always_inline)) -> int64_t {
    if constexpr (!PAGED) return rowbase;
    else return page_row(npg > 64 ? table(j) : __builtin_amdgcn_readlane(pg_lane, j >> prs), j);
  };
  auto rel_lane = [&](int j) __attribute__((always_inline)) -> int64_t {
    if constexpr (!PAGED) return rowbase;
    else return page_row(npg > 64 ? table(j) : __shfl(pg_lane, j >> prs), j);
  };
  const int g = Q4 ? (32 * qd) / 64 : 0;
  const uint32_t lane_off = 16 * qd, lane_soff = 4 * g;
  const DqConst dq{0x000F000Fu, 0x00F000F0u, in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
  DecQuery<D, Q4> Q;
  Q.load(a.qkv + (int64_t)r * 3 * a.h1 + h * D + (Q4 ? 32 : 8) * qd);

  // ---- pass 1: scores
  // rows past the visible range are clamped to its last row; the rows of one
  // load stay in the page of its first row (or of that last row)
  auto load_k = [&](DecPart<UK, Q4>& X, int c) {
    int row[UK];
    int64_t rel[UK];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      row[u] = min(c * CRK + rho + RPI * u, T - 1);
      rel[u] = rel_uniform(min(c * CRK + RPI * u, T - 1));
    }
    load_rows<D, Q4>(X, kb, ksb, rel, row, lane_off, lane_soff);
  };
  auto score = [&](const DecPart<UK, Q4>& X, int c) {
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const float t = row_score<D, Q4>(X.c[u], Q4 ? X.sm[u] : 0u, Q, dq);
      const int row = c * CRK + rho + RPI * u;
      if (qd == 0 && row < T) sc[row] = t;
    }
  };
  {
    const int nc = (T + CRK - 1) / CRK;
    DecPart<UK, Q4> XA, XB;
    load_k(XA, 0);
    if (nc > 1) load_k(XB, 1);
    for (int c = 0; c < nc; c += 2) {
      score(XA, c);
      if (c + 2 < nc) load_k(XA, c + 2);
      if (c + 1 < nc) {
        score(XB, c + 1);
        if (c + 3 < nc) load_k(XB, c + 3);
      }
    }
  }
  __syncthreads();

  // ---- pass 2: exact Top-K
  // Slots past the visible rows hold key 0; every candidate below has a bit
  // set, so they are never counted.  Up to 32 slots per lane the keys stay
  // in registers; beyond that each round re-reads them from LDS.
  constexpr int NR = NS <= 32 ? NS : 1;
  const int nsl = (T + 63) / 64;
  uint32_t key[NR];
  float mloc = -INFINITY;
  if constexpr (NS <= 32) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = 64 * s + lane;
      const float z = j < T ? sc[j] : -INFINITY;
      key[s] = j < T ? score_key(z) : 0u;
      mloc = fmaxf(mloc, z);
    }
  } else {
    for (int j = lane; j < T; j += 64) mloc = fmaxf(mloc, sc[j]);
  }
  const float zmax = wave_max_dpp(mloc);
  auto count_at_least = [&](uint32_t cand) {  // this lane's keys >= cand (cand > 0)
    int cnt = 0;
    if constexpr (NS <= 32) {
#pragma unroll
      for (int s = 0; s < NS; ++s) cnt += key[s] >= cand ? 1 : 0;
    } else {
      for (int j = lane; j < T; j += 64) cnt += score_key(sc[j]) >= cand ? 1 : 0;
    }
    return cnt;
  };
  // tau: the K-th largest key, or any value with exactly K keys at or above
  // it (the kept set is then settled and the search stops early)
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    const int cnt = wave_total(count_at_least(cand));
    if (cnt >= K) {
      tau = cand;
      if (cnt == K) break;
    }
  }
  // rows above tau (none if tau is the largest key), then ties at tau, lowest
  // rows first, until exactly K rows are kept
  const int need = K - (tau == 0xFFFFFFFFu ? 0 : wave_total(count_at_least(tau + 1u)));
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0, ties = 0;
  int32_t* idx = a.idx ? a.idx + ((int64_t)r * a.H + h) * K : nullptr;
  for (int s = 0; s < nsl; ++s) {  // keys re-derived from LDS: a plain loop
    const int j = 64 * s + lane;
    const bool valid = j < T;
    const uint32_t kj = valid ? score_key(sc[j]) : 0u;
    const bool eq = valid && kj == tau;
    const uint64_t em = __ballot(eq);
    const bool take = (valid && kj > tau) || (eq && ties + __popcll(em & below) < need);
    ties += __popcll(em);
    const uint64_t tm = __ballot(take);
    if (take) {
      const int at = base + __popcll(tm & below);
      sel[at] = j;
      if (idx && at < K) idx[at] = j;
    }
    base += __popcll(tm);
  }
  __syncthreads();

  // ---- pass 3: the kept V rows
  const float c2 = 1.44269504088896341f / sqrtf((float)D);  // exp(x / sqrt(D)) = exp2(x c2)
  const float mc = -zmax * c2;
  DecAcc<D, Q4> A;
  float l_lane = 0.f;
  auto load_v = [&](DecPart<UV, Q4>& X, float (&z)[UV], int c) {
    int row[UV];
    int64_t rel[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int e = c * CRV + rho + RPI * u;
      row[u] = sel[min(e, K - 1)];
      z[u] = e < K ? sc[row[u]] : -INFINITY;  // list slots past K weigh 0
      rel[u] = rel_lane(row[u]);
    }
    load_rows<D, Q4>(X, vb, vsb, rel, row, lane_off, lane_soff);
  };
  auto accumulate = [&](const DecPart<UV, Q4>& X, const float (&z)[UV]) {
    float p[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      p[u] = __builtin_amdgcn_exp2f(fmaf(z[u], c2, mc));
      l_lane += p[u];
    }
    A.add(X, p, dq);
  };
  {
    const int nc = (K + CRV - 1) / CRV;
    DecPart<UV, Q4> VA, VB;
    float zA[UV], zB[UV];
    load_v(VA, zA, 0);
    if (nc > 1) load_v(VB, zB, 1);
    for (int c = 0; c < nc; c += 2) {
      accumulate(VA, zA);
      if (c + 2 < nc) load_v(VA, zA, c + 2);
      if (c + 1 < nc) {
        accumulate(VB, zB);
        if (c + 3 < nc) load_v(VB, zB, c + 3);
      }
    }
  }
  A.finish(l_lane, rho, a.out + (int64_t)r * a.h1 + h * D + (Q4 ? 32 : 8) * qd);
}

// Largest visible row count the kernel takes (score and list slots in LDS).
constexpr int TOPK_MAX_T = 4096;

hp_status launch_topk_attention(int32_t b, int32_t h1, int32_t heads, const void* qkv, int32_t pos,
                                const int32_t* dpos, int32_t max_t, int32_t topk, const hp_kv& kv,
                                void* out, int32_t* idx, hipStream_t st, const int32_t* rpos) {
  if (max_t < 1 || max_t > TOPK_MAX_T) return HP_ERR_SHAPE;
  const int D = h1 / heads;
  const bool paged = kv.page_rows > 0;
  TopkArgs a{(const _Float16*)qkv, h1,   heads, pos,  dpos, topk,
             kv.cap,               kv.k, kv.v,  (const uint32_t*)kv.k_sm,
             (const uint32_t*)kv.v_sm, (_Float16*)out, idx, rpos,
             paged ? kv.pages : nullptr, kv.page_rows, kv.pool_pages};
  const dim3 grid((unsigned)((int64_t)b * heads));
  Prof prof(kv.fmt == HP_Q4 ? "attn_topk_q4" : "attn_topk_f16", st);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(64), 0, st, a); };
  auto by_ns = [&](auto d, auto q4) {
    constexpr int DD = decltype(d)::value;
    constexpr bool QQ = decltype(q4)::value;
    auto pick = [&](auto kc, auto kp) { paged ? go(kp) : go(kc); };
    if (max_t <= 256) pick(k_topk_attn<DD, QQ, 4, false>, k_topk_attn<DD, QQ, 4, true>);
    else if (max_t <= 512) pick(k_topk_attn<DD, QQ, 8, false>, k_topk_attn<DD, QQ, 8, true>);
    else if (max_t <= 768) pick(k_topk_attn<DD, QQ, 12, false>, k_topk_attn<DD, QQ, 12, true>);
    else if (max_t <= 1024) pick(k_topk_attn<DD, QQ, 16, false>, k_topk_attn<DD, QQ, 16, true>);
    else if (max_t <= 1536) pick(k_topk_attn<DD, QQ, 24, false>, k_topk_attn<DD, QQ, 24, true>);
    else if (max_t <= 2048) pick(k_topk_attn<DD, QQ, 32, false>, k_topk_attn<DD, QQ, 32, true>);
    else if (max_t <= 3072) pick(k_topk_attn<DD, QQ, 48, false>, k_topk_attn<DD, QQ, 48, true>);
    else pick(k_topk_attn<DD, QQ, 64, false>, k_topk_attn<DD, QQ, 64, true>);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using QT = std::true_type;
  using QF = std::false_type;
  if (D == 128) kv.fmt == HP_Q4 ? by_ns(I128{}, QT{}) : by_ns(I128{}, QF{});
  else kv.fmt == HP_Q4 ? by_ns(I64{}, QT{}) : by_ns(I64{}, QF{});
  return HP_OK;
}

}  // namespace hp
