// KV-cache append and attention for the FlexGen layer ([FlexGen] paper
// notes, background section: prefill and decode equations; section 5: the KV
// cache is stored as int4 groups of 64 along the hidden dimension and
// converted back before use; [SpecPipe] 2.2.1-2.2.2: tree masks).
//
// Decode attention is HBM-bound (about 1 flop per byte of packed cache), so
// it runs on the vector ALUs, one wave per (request, head, query), streaming
// the cache in chunks with the row slices, scores and value sums of
// decode_dev.h; the loads are non-temporal and the next chunk's K (V) is
// requested as soon as the current chunk's scores (values) are formed; the
// softmax is online over chunks with DPP reductions.
// Multi-query decode (tree tokens) and prefill attention run on MFMA; see
// their sections below.
#include <math.h>

#include "common.h"
#include "decode_dev.h"
#include "dequant_dev.h"
#include "lds_dma.h"
#include "quant_dev.h"

namespace hp {

// ------------------------------------------------------------ KV append
// Per-token form (decode steps, ragged or paged appends, d = 64, fp16
// caches; whole 16-row chunks of a contiguous int4 cache with d = 128 go to
// k_kv_append_tile below): a workgroup codes 32 AU groups of 64 channels of
// one new token's K | V columns (2 h1 contiguous halves: a wave reads 1 KB
// contiguous; a lane codes AU groups, their loads issued first) and writes
// each group into the head-major cache row of its head.  Neighbouring rows of
// one head share cache lines, so the workgroups of 16 consecutive tokens are
// given ids of one residue mod 8 (workgroup ids reach the 8 XCDs round-robin)
// and write those lines through one XCD's L2.  Their 8-byte scale/min pieces
// still reach memory as partial writes (1.3x the written bytes at the
// prefill shapes), which is what the tiled form avoids.
struct AppendArgs {
  const _Float16* qkv;
  int b, q, h1, H, D, pos;
  const int32_t* dpos;
  const int32_t* rpos;  // per-request first row (clamped to [0, pos]), or NULL
  int cap;
  void* k;
  void* v;
  uint32_t* ksm;
  uint32_t* vsm;
  const int32_t* pages;  // paged cache: page table [b][cap / PR], or NULL
  int PR, pool;          // rows per page (a power of two), pages in the pool
};

// Physical cache row (in rows of one head) of logical row j of request r,
// head h: contiguous [b][H][cap], or paged [page][H][PR] through the table
// (PR a power of two: shifts, not divisions).
__device__ __forceinline__ int64_t cache_row(const int32_t* pages, int PR, int pool, int cap,
                                             int H, int r, int h, int j) {
  if (!pages) return ((int64_t)r * H + h) * cap + j;
  const int sh = __builtin_ctz(PR);
  const int pg = min(max(pages[(int64_t)r * (cap >> sh) + (j >> sh)], 0), pool - 1);
  return ((int64_t)pg * H + h) * PR + (j & (PR - 1));
}

constexpr int AU = 4;

template <bool Q4, int D>
__global__ __launch_bounds__(256) void k_kv_append(AppendArgs a) {
  constexpr int G = D / 64;  // groups per head row
  const int sub = threadIdx.x & 7;
  const int HG = a.H * G;    // groups of K (and of V) per token
  const int SC = (2 * HG + 32 * AU - 1) / (32 * AU);  // workgroups per token
  // id -> (chunk of 16 tokens, token, span piece): the 16 SC workgroups of a
  // chunk are the ids x, x + 8, x + 16, ... of one residue x
  const int id = blockIdx.x, x = id & 7, k = id >> 3;
  const int per = 16 * SC;
  const int chunk = x + 8 * (k / per), within = k % per;
  const int token = chunk * 16 + within / SC, sc = within % SC;  // token = r * q + i
  if (token >= a.b * a.q) return;
  const int r = token / a.q, i = token % a.q;
  const int pos = a.rpos ? min(max(a.rpos[r], 0), a.pos) : a.pos + (a.dpos ? *a.dpos : 0);
  const _Float16* src = a.qkv + (int64_t)token * 3 * a.h1 + a.h1;  // K | V of this token
  const int gg0 = sc * (32 * AU) + (threadIdx.x >> 3);
  uint4 raw[AU];
#pragma unroll
  for (int u = 0; u < AU; ++u) {
    const int gg = gg0 + 32 * u;
    if (gg < 2 * HG) raw[u] = stream_load16((const uint4*)(src + 64 * gg) + sub);
  }
#pragma unroll
  for (int u = 0; u < AU; ++u) {
    const int gg = gg0 + 32 * u;
    if (gg >= 2 * HG) continue;  // the same for the 8 lanes of a group
    const int which = gg >= HG;  // 0 = K, 1 = V
    const int hg = gg - which * HG;
    const int h = hg / G, g = hg % G;
    const int64_t row = cache_row(a.pages, a.PR, a.pool, a.cap, a.H, r, h, pos + i);
    if constexpr (Q4) {
      uint32_t smw;
      const uint32_t word = quant_group8(raw[u], smw);
      uint8_t* dst = (uint8_t*)(which ? a.v : a.k) + row * (D / 2) + 32 * g;
      *(uint32_t*)(dst + 4 * sub) = word;
      if (sub == 0) (which ? a.vsm : a.ksm)[row * G + g] = smw;
    } else {
      _Float16* dst = (_Float16*)(which ? a.v : a.k) + row * D + 64 * g;
      *(uint4*)(dst + 8 * sub) = raw[u];
    }
  }
}

// Tiled int4 append for whole chunks of rows (prefill and multi-token
// appends into a contiguous cache, d = 128, rows starting at a multiple of
// 16): one workgroup per (request, 16 consecutive tokens, 4 heads).  The
// 8 lanes of a group code it as k_kv_append does (the same coder, the same
// bits).  Group (slot u, wave w, octet j): tile (head, K or V) = (4 u + w) / 4,
// rows 4 ((4 u + w) % 4) + j / 2 of the chunk, group j % 2 of the row, so one
// store instruction writes 4 consecutive cache rows of one head: 256
// contiguous bytes of codes.  The scale/min words of a tile (16 rows x 2
// groups, 128 contiguous bytes in the cache) meet in LDS in cache order and
// leave as 16-byte stores: every memory write covers whole 64-byte pieces, so
// none needs the memory's read-modify-write of a partial piece.
constexpr int KT_ROWS = 16, KT_HEADS = 4;
constexpr int KT_SLOTS = 2 * KT_HEADS;  // (heads x (K, V) x 4 row quads) / 4 waves groups per lane

__global__ __launch_bounds__(256) void k_kv_append_tile(AppendArgs a) {
  __shared__ uint32_t sml[4 * KT_SLOTS][8];  // [tile * 4 + row quad][octet]: cache order per tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane >> 3, sub = lane & 7;
  const int nhb = (a.H + KT_HEADS - 1) / KT_HEADS, nch = (a.q + KT_ROWS - 1) / KT_ROWS;
  const int hb = blockIdx.x % nhb, rc = blockIdx.x / nhb;
  const int c = rc % nch, r = rc / nch;
  const int i0 = c * KT_ROWS;
  uint4 raw[KT_SLOTS];
#pragma unroll
  for (int u = 0; u < KT_SLOTS; ++u) {
    const int idx = 4 * u + w;
    const int h = hb * KT_HEADS + (idx >> 3), which = (idx >> 2) & 1;
    const int i = i0 + 4 * (idx & 3) + (j >> 1);
    const int ii = min(i, a.q - 1), hh = min(h, a.H - 1);  // rows and heads past the end re-read
    const _Float16* src = a.qkv + ((int64_t)r * a.q + ii) * 3 * a.h1 + (int64_t)a.h1 * (1 + which) +
                          hh * 128 + 64 * (j & 1);
    raw[u] = stream_load16((const uint4*)src + sub);
  }
#pragma unroll
  for (int u = 0; u < KT_SLOTS; ++u) {
    const int idx = 4 * u + w;
    const int h = hb * KT_HEADS + (idx >> 3), which = (idx >> 2) & 1;
    const int i = i0 + 4 * (idx & 3) + (j >> 1);
    uint32_t smw;
    const uint32_t word = quant_group8(raw[u], smw);
    if (sub == 0) sml[idx][j] = smw;
    if (i < a.q && h < a.H) {
      const int64_t row = ((int64_t)r * a.H + h) * a.cap + a.pos + i;
      uint8_t* dst = (uint8_t*)(which ? a.v : a.k) + row * 64 + 32 * (j & 1);
      __builtin_nontemporal_store(word, (uint32_t*)(dst + 4 * sub));  // streamed out
    }
  }
  __syncthreads();
  if (threadIdx.x < 16 * KT_HEADS) {
    // 2 KT_HEADS tiles x 128 bytes: thread -> tile t / 8, bytes 16 (t % 8) ..
    // +15 (rows 2 (t % 8) and 2 (t % 8) + 1 of the chunk)
    const int tile = threadIdx.x >> 3, part = threadIdx.x & 7;
    const int h = hb * KT_HEADS + (tile >> 1), which = tile & 1;
    const int i = i0 + 2 * part;
    if (h < a.H && i < a.q) {
      const uint32_t* s4 = &sml[4 * tile + (part >> 1)][4 * (part & 1)];
      const int64_t row = ((int64_t)r * a.H + h) * a.cap + a.pos + i;
      uint32_t* dst = (which ? a.vsm : a.ksm) + row * 2;
      if (i + 1 < a.q) {
        *(uint4*)dst = make_uint4(s4[0], s4[1], s4[2], s4[3]);
      } else {
        dst[0] = s4[0];
        dst[1] = s4[1];
      }
    }
  }
}

// ------------------------------------------------------- decode attention
struct DecArgs {
  const _Float16* qkv;
  int q, h1, H, pos;
  const int32_t* dpos;
  const int32_t* plen;  // per-request prefix lengths (clamped to [0, pos]), or NULL
  const uint64_t* masks;
  int cap;
  const void* k;
  const void* v;
  const uint32_t* ksm;
  const uint32_t* vsm;
  _Float16* out;
  const int32_t* pages;  // paged cache (streaming kernel only), or NULL
  int PR, pool;
};
// Cache rows before the new tokens of request r: the same for every request
// (pos, plus the step counter of a replayed graph), or per request.
__device__ __forceinline__ int prefix_len(const DecArgs& a, int r) {
  if (a.plen) return min(max(a.plen[r], 0), a.pos);
  return a.pos + (a.dpos ? *a.dpos : 0);
}

// A chunk of an int4 cache is 3 loads (133 VGPRs, 3 waves per SIMD: the
// extra rows in flight outweigh the lower occupancy, 3-9% at the 30B decode
// shape against 2 loads).  PG: 0 = rows contiguous per (request, head);
// 1 = a paged cache of at most 64 pages per request, their numbers held in
// lanes; 2 = more pages, the table read from memory per load (one page per
// load either way).
template <int D, bool Q4, bool MASKED, int PG>
__global__ __launch_bounds__(64) void k_decode_attn(DecArgs a) {
  constexpr bool PAGED = PG > 0;
  using S = DecShape<D, Q4>;
  constexpr int LPR = S::LPR, RPI = S::RPI, RB = S::RB, G = S::G;
  // a chunk is U loads of RPI rows for K and for V; the next chunk is loaded
  // while the current one is computed
  constexpr int U = Q4 ? 3 : 4, CR = U * RPI;
  const int lane = threadIdx.x;
  const int qd = lane % LPR, rho = lane / LPR;
  const int i = blockIdx.x % a.q;
  const int rh = blockIdx.x / a.q;
  const int h = rh % a.H, r = rh / a.H;
  const int P = prefix_len(a, r);
  const int R = MASKED ? P + a.q : P + i + 1;
  const uint64_t mask = MASKED ? a.masks[(int64_t)r * a.q + i] : 0ull;
  // wave-uniform bases, per-lane 32-bit byte offsets.  The rows of one load
  // (RPI rows from a multiple of RPI, RPI | 64 | PR) lie in one page of a
  // paged cache: base(j) is the physical row of logical row j less j, so
  // every logical row of that load is at base(j) + row (rows clamped to the
  // last visible one stay in its page: the clamp only applies within the
  // load that holds that row, or to loads past it, whose j is that row).
  const int64_t rowbase = ((int64_t)r * a.H + h) * a.cap;
  // paged: the request's page numbers (up to 64) sit one per lane, loaded
  // once, so a load's page comes from a lane read instead of a table load
  // the cache load would have to wait for
  const int prs = PAGED ? __builtin_ctz(a.PR) : 0;  // page rows are a power of two
  const int npg = PAGED ? a.cap >> prs : 0;
  int pg_lane = 0;
  if constexpr (PG == 1) {
    if (lane < npg) pg_lane = min(max(a.pages[(int64_t)r * npg + lane], 0), a.pool - 1);
  }
  auto base = [&](int j) __attribute__((always_inline)) -> int64_t {
    if constexpr (PG == 0) return rowbase;
    else if constexpr (PG == 2) return cache_row(a.pages, a.PR, a.pool, a.cap, a.H, r, h, j) - j;
    else {
      const int jp = j >> prs;  // the page slot of row j: base = (page's first row) - (jp PR)
      const int pg = __builtin_amdgcn_readlane(pg_lane, jp);
      return ((int64_t)pg * a.H + h - jp) * a.PR;
    }
  };
  const int g = Q4 ? (32 * qd) / 64 : 0;  // int4 group of this lane's dims
  const uint32_t lane_off = 16 * qd, lane_soff = 4 * g;
  // exp(x / sqrt(D)) = exp2(x * c2)
  const float c2 = 1.44269504088896341f / sqrtf((float)D);

  const DqConst dq{0x000F000Fu, 0x00F000F0u, in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
  DecQuery<D, Q4> Q;
  Q.load(a.qkv + ((int64_t)r * a.q + i) * 3 * a.h1 + h * D + (Q4 ? 32 : 8) * qd);
  DecAcc<D, Q4> A;
  float m_run = -INFINITY, l_lane = 0.f;

  // rows past the visible range are clamped to its last row (their weight is 0)
  auto load = [&](DecPart<U, Q4>& X, const void* cache, const uint32_t* smc, int c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t bu = base(min(c * CR + RPI * u, R - 1));
      const uint8_t* cb = (const uint8_t*)cache + bu * RB;
      const uint8_t* sb = (const uint8_t*)(smc + bu * G);
      const uint32_t row = (uint32_t)min(c * CR + rho + RPI * u, R - 1);
      // the cache is streamed once per step: non-temporal loads keep it from
      // displacing reusable lines in the caches
      X.c[u] = __builtin_nontemporal_load((const u32x4*)(cb + (row * RB + lane_off)));
      if constexpr (Q4) X.sm[u] = *(const uint32_t*)(sb + (row * (4 * G) + lane_soff));
    }
    // keeps the compiler from merging this load with the one of the previous
    // iteration into a load at the loop head (which would undo the prefetch)
    asm volatile("" ::: "memory");
  };

  // K and V of a chunk are loaded into one register set each; the next
  // chunk's K is requested as soon as the scores are formed and its V as soon
  // as the values are accumulated, so each stream is in flight while the
  // other phase computes.
  DecPart<U, Q4> K, V;
  const int nc = (R + CR - 1) / CR;
  load(K, a.k, a.ksm, 0);
  load(V, a.v, a.vsm, 0);
  for (int c = 0; c < nc; ++c) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float t = row_score<D, Q4>(K.c[u], Q4 ? K.sm[u] : 0u, Q, dq);
      const int row = c * CR + rho + RPI * u;
      bool valid = row < R;
      if constexpr (MASKED)
        valid = valid & ((row < P) | (bool)((mask >> ((unsigned)(row - P) & 63u)) & 1ull));
      s[u] = valid ? t : -INFINITY;
    }
    load(K, a.k, a.ksm, c + 1);
    // online softmax (chunk max is wave-uniform)
    float cm = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[u]);
    cm = wave_max_dpp(cm);
    const float m_new = fmaxf(m_run, cm);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float mc = -m_use * c2;
    const float alpha = __builtin_amdgcn_exp2f(fmaf(m_run, c2, mc));
    m_run = m_new;
    float p[U], ps = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u] = __builtin_amdgcn_exp2f(fmaf(s[u], c2, mc));
      ps += p[u];
    }
    l_lane = fmaf(l_lane, alpha, ps);
    if (alpha != 1.f) A.rescale(alpha);
    A.add(V, p, dq);
    load(V, a.v, a.vsm, c + 1);
  }
  A.finish(l_lane, rho, a.out + ((int64_t)r * a.q + i) * a.h1 + h * D + (Q4 ? 32 : 8) * qd);
}

// ------------------------------------------------------ prefill attention
// Causal attention over the fresh fp16 K/V of the prompt (query i sees keys
// 0..i), on MFMA (v_mfma_f32_16x16x32_f16), flash-attention style.
//  * Workgroup = 4 waves = 64 queries of one (request, head); wave w owns
//    queries 16 w .. 16 w + 15.  Key blocks of 64 rows of K and V go to LDS
//    by direct loads (double-buffered) and serve all 4 waves.
//  * Scores S^T = K Q^T: operand A = 16 keys x 32 dims of K (one 16-byte
//    LDS read per lane; 16-byte chunks XOR-swizzled by key), operand B = the
//    wave's Q fragments, held in registers.  Lane l then holds 16 scores of
//    query l % 16, so the online-softmax state is per lane.
//  * The key rows of each 16-key score tile are permuted so that lane group
//    l / 16 ends up with 8 consecutive keys per 32-key step: exactly the
//    operand-B layout of the value product.
//  * Output O^T = V^T P^T: operand A = 16 dims x 32 keys of V^T, read with
//    the transposing LDS read ds_read_b64_tr_b16 (two reads of 4 keys; V's
//    chunks are XOR-swizzled so the 4 rows of one read hit distinct banks),
//    operand B = the probabilities as binary16; lane l accumulates 4 dims
//    of query l % 16 per 16-dim block.
constexpr int PF_QB = 64;  // queries per workgroup
constexpr int PF_KB = 64;  // keys per block

struct PfArgs {
  const _Float16* qkv;
  int s, h1, H;
  _Float16* out;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 ds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) void*)p);
}

// Chunk swizzles of the fp16 K and V tiles (SPR 16-byte slots per row): the
// 16 keys of a score tile, and the 4 rows of one transposing read, fall in
// distinct banks.
template <int SPR>
__device__ __forceinline__ int swz_k(int key) {
  return ((key & 3) | (((key >> 3) & 3) << 2)) & (SPR - 1);
}
template <int SPR>
__device__ __forceinline__ int swz_v(int key) {
  return ((key & 3) << 1) & (SPR - 1);
}

// One block of 64 keys for the 16 queries of a wave (query l % 16 per lane):
// scores S^T = K Q^T, keys with !visible(kidx) masked, online softmax, and
// O^T += V^T P^T.  Kl, Vl: fp16 tiles of the block (64 rows of 2 D bytes);
// VK: the V tile uses the K tile's chunk swizzle (the transposing reads
// measured as fast with either).
template <int D, bool VK = false, class Vis>
__device__ __forceinline__ void flash_block(const uint8_t* Kl, const uint8_t* Vl,
                                            const f16x8 (&qf)[D / 32], int k0, Vis visible,
                                            float c2, float& m_run, float& l_lane,
                                            f32x4 (&o)[D / 16]) {
  constexpr int KS = D / 32, DB = D / 16, RB = 2 * D, SPR = RB / 16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, G = lane >> 4;
  // scores of 4 tiles of 16 keys; tile T row m holds key
  // 32 (T / 2) + 8 (m / 4) + 4 (T % 2) + m % 4
  f32x4 sc[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int key = 32 * (T / 2) + 8 * (r16 / 4) + 4 * (T % 2) + (r16 % 4);
    const uint8_t* kr = Kl + key * RB;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 kf = *(const f16x8*)(kr + 16 * ((G + 4 * ks) ^ swz_k<SPR>(key)));
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ks], c, 0, 0, 0);
    }
    sc[T] = c;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!visible(k0 + 32 * (T / 2) + 8 * G + 4 * (T % 2) + e)) sc[T][e] = -INFINITY;
      mx = fmaxf(mx, sc[T][e]);
    }
  mx = max_xor32(max_xor16(mx));
  // The running maximum moves only when a score exceeds it by more than 8 in
  // the exponent (base 2), so the rescale of l and O is rare after the first
  // blocks; the probabilities, up to 2^8, stay well inside binary16 and the
  // final division by l removes the common factor.  (The first finite
  // maximum always moves it: -inf compares as an unbounded rise; an all-
  // masked lane, -inf to -inf, compares false and keeps probabilities 0.)
  const float m_new = fmaxf(m_run, mx);
  if (__any((m_new - m_run) * c2 > 8.f)) {
    const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c2);
    m_run = m_new;
    l_lane *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
  }
  const float mc = -(m_run == -INFINITY ? 0.f : m_run) * c2;
  float ps = 0.f;
  f16x8 pb[2];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[T][e], c2, mc));
      ps += p;
      pb[T / 2][4 * (T % 2) + e] = (_Float16)p;
    }
  l_lane += ps;
  // O^T += V^T P^T over two 32-key steps
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f16x8 vf;
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        const int row = 32 * p + 8 * G + 4 * n2 + r16 / 4;
        const int d = 16 * db + 4 * (r16 % 4);
        const uint8_t* vp = Vl + row * RB + 16 * ((d / 8) ^ (VK ? swz_k<SPR>(row) : swz_v<SPR>(row))) + 2 * (d % 8);
        const f16x4 th = __builtin_bit_cast(f16x4, ds_read_tr16(vp));
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[4 * n2 + e] = th[e];
      }
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[p], o[db], 0, 0, 0);
    }
  }
}

// Normalised output of a wave's 16 queries: lane l holds tile positions
// 16 db + 4 (l / 16) + e.  PERM: the V tile stores each 8-dim chunk in the
// order 0 4 1 5 2 6 3 7 (the int4 expansion's natural order), so a lane with
// l / 16 even holds dims {0, 4, 1, 5} of its chunk and the lane 16 above it
// dims {2, 6, 3, 7}; the pair swaps two values to write dims in order.
template <int D, bool PERM = false>
__device__ __forceinline__ void flash_store(_Float16* row, float l_lane, const f32x4 (&o)[D / 16]) {
  const int G = (threadIdx.x & 63) >> 4;
  // the 4 lanes of a query hold complementary key subsets: total their sums
  const float l = sum_xor32(sum_xor16(l_lane));
  const float inv = 1.0f / l;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    f16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (_Float16)(o[db][e] * inv);
    if constexpr (PERM) {
      // even G sends dims 4, 5 (y1, y3) and receives 2, 3; odd G the reverse
      const bool odd = G & 1;
      const f16x2 send = odd ? f16x2{y[0], y[2]} : f16x2{y[1], y[3]};
      const f16x2 got = h2_of(__shfl_xor(__builtin_bit_cast(uint32_t, send), 16));
      y = odd ? f16x4{got[0], got[1], y[1], y[3]} : f16x4{y[0], y[2], got[0], got[1]};
    }
    if (row) *(f16x4*)(row + 16 * db + 4 * G) = y;
  }
}

// Two workgroups per CU (the LDS ring holds 64 KB at D = 128): the bound
// caps a lane at 256 registers, so the output accumulators stay in VGPRs
// (with 512 the compiler put them in AGPRs and moved them through VGPRs for
// every rescale).
template <int D>
__global__ __launch_bounds__(256, 2) void k_prefill_attn(PfArgs a) {
  constexpr int KS = D / 32;           // k-steps of the score product
  constexpr int DB = D / 16;           // 16-dim output blocks
  constexpr int RB = 2 * D;            // bytes per key row in LDS
  constexpr int SPR = RB / 16;         // 16-byte slots per row
  constexpr int KPI = 64 / SPR;        // key rows per direct load (1 KB)
  constexpr int NI = PF_KB / KPI / 4;  // direct loads per wave per block, for K and for V
  constexpr int STAGE = 2 * PF_KB * RB;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int lane = threadIdx.x & 63, r16 = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = a.s;
  const int nqb = (s + PF_QB - 1) / PF_QB;
  // Workgroup ids go to the 8 XCDs round-robin (id % 8), each XCD with its
  // own L2: the query blocks of one (request, head) run in consecutive turns
  // of one XCD, so their common K/V prefix is fetched from HBM once there.
  const int nrh = (int)gridDim.x / nqb, full = (nrh / 8) * 8 * nqb, id = blockIdx.x;
  int rh, jq;
  if (id < full) {
    const int t = id / 8;
    rh = 8 * (t / nqb) + id % 8;
    jq = t % nqb;
  } else {
    rh = (nrh / 8) * 8 + (id - full) / nqb;
    jq = (id - full) % nqb;
  }
  const int qb = nqb - 1 - jq;  // longest query blocks first
  const int h = rh % a.H, r = rh / a.H;
  const int64_t ld = 3LL * a.h1;
  const _Float16* base = a.qkv + (int64_t)r * s * ld + h * D;
  const int qi = qb * PF_QB + 16 * wave + r16;  // this lane's query
  const float c2 = 1.44269504088896341f / sqrtf((float)D);

  // Q fragments (operand B of the score product): dims 8 G + 32 ks .. +7
  f16x8 qf[KS];
  {
    const _Float16* qp = base + (int64_t)min(qi, s - 1) * ld + 8 * G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const f16x8*)(qp + 32 * ks);
  }

  const uint32_t lbase = lds_off(lds);
  const int nkb = min(qb + 1, (s + PF_KB - 1) / PF_KB);
  auto issue = [&](int kb, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int u = wave * NI + i;
      const int key = KPI * u + lane / SPR;  // key within the block
      const int slot = lane % SPR;
      const int row = min(kb * PF_KB + key, s - 1);
      const _Float16* src = base + (int64_t)row * ld;
      dma16(src + a.h1 + 8 * (slot ^ swz_k<SPR>(key)),
            __builtin_amdgcn_readfirstlane(lbase + st * STAGE + u * 1024));
      dma16(src + 2 * a.h1 + 8 * (slot ^ swz_v<SPR>(key)),
            __builtin_amdgcn_readfirstlane(lbase + st * STAGE + PF_KB * RB + u * 1024));
    }
  };

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  auto visible = [&](int kidx) __attribute__((always_inline)) { return kidx <= qi && kidx < s; };
  auto all_visible = [](int) __attribute__((always_inline)) { return true; };

  auto block = [&](int kb, auto vis) __attribute__((always_inline)) {
    const int st = kb & 1;
    wait_vm<0, 0>();
    __builtin_amdgcn_s_barrier();
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    const uint8_t* Kl = lds + st * STAGE;
    flash_block<D>(Kl, Kl + PF_KB * RB, qf, kb * PF_KB, vis, c2, m_run, l_lane, o);
  };
  // blocks left of the diagonal are visible to every query of the group (no
  // per-key mask), then the diagonal block
  issue(0, 0);
  int kb = 0;
  for (; kb < nkb - 1; ++kb) block(kb, all_visible);
  block(kb, visible);
  wait_vm<0>();
  flash_store<D>(qi < s ? a.out + ((int64_t)r * s + qi) * a.h1 + h * D : nullptr, l_lane, o);
}

// ------------------------------------------------ multi-query decode (int4)
// q >= 16 new tokens per request over the int4 cache (tree decode of
// [SpecPipe] 2.2.1, or chain decode): one workgroup per (request, head),
// 4 waves of 16 queries.  Each 64-row block of the cache is expanded once
// into fp16 K and V tiles (fp16(c * scale + min), one rounding: the values
// the oracle's dequantiser gives), and flash_block runs over the tiles with
// the tree visibility: every prefix row, plus tree rows flagged in the
// query's mask (or rows up to the query's own for a chain).  Pipelined: the
// codes of block kb + 1 come to registers one block ahead, the tiles are
// double-buffered, and in one phase each wave expands block kb + 1 into the
// free tile buffer and runs the block step of block kb on the other (one
// barrier per block, no branch between the two, so the expansion's vector
// work can interleave with the step's MFMAs; 84-88 -> 71-78 us on the tree
// workload against a form with a staging ring, an expansion phase and a
// step phase).
template <int D>
__global__ __launch_bounds__(256, 2) void k_multi_attn(DecArgs a) {
  constexpr int KS = D / 32, RB = 2 * D, SPR = RB / 16;
  constexpr int CB = D / 2;          // code bytes per cache row
  constexpr int NG = D / 64;         // groups per row
  constexpr int PPR = CB / 16;       // 16-byte pieces per row
  constexpr int NP = 2 * 16 * PPR / 64;  // (tensor, row, piece) units per lane and block
  constexpr int TILE = 2 * 64 * RB;  // K and V tiles of one block
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[2 * TILE];

  const int lane = threadIdx.x & 63, r16 = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % a.H, r = blockIdx.x / a.H;
  const int P = prefix_len(a, r);
  const int R = P + a.q;
  const int qi = 16 * wave + r16;
  const int qrow = min(qi, a.q - 1);
  const uint64_t mask = a.masks ? a.masks[(int64_t)r * a.q + qrow] : 0ull;
  const float c2 = 1.44269504088896341f / sqrtf((float)D);
  const int64_t rowbase = ((int64_t)r * a.H + h) * a.cap;
  const uint8_t* kc = (const uint8_t*)a.k + rowbase * CB;
  const uint8_t* vc = (const uint8_t*)a.v + rowbase * CB;
  const uint32_t* ks_ = a.ksm + rowbase * NG;
  const uint32_t* vs_ = a.vsm + rowbase * NG;

  // Q fragments in the tiles' dim order (each 8-dim chunk as 0 4 1 5 2 6 3 7)
  f16x8 qf[KS];
  {
    const _Float16* qp = a.qkv + ((int64_t)r * a.q + qrow) * 3 * a.h1 + h * D + 8 * G;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const f16x8 v = *(const f16x8*)(qp + 32 * k);
      qf[k] = f16x8{v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};
    }
  }

  // this wave's units of a block: rows 16 wave .. 16 wave + 15 of K and V,
  // unit u = 64 p + lane -> tensor, row, 16-byte piece
  // unit rem of a tensor: row and 16-byte piece.  With 4 pieces per row,
  // 16 consecutive lanes take pieces 0..3 of 4 consecutive rows (4 rows per
  // piece), so each 8-lane group of a tile write covers 4 rows x 2 pieces:
  // with the K swizzle (used for both tiles here) their 16-byte slots fall in
  // distinct banks.  Rows 0..3 x pieces 0..3 are still one contiguous 256 B
  // of the cache for the loads.
  auto urow = [](int rem) { return PPR == 4 ? (rem & 3) + 4 * (rem >> 4) : rem / PPR; };
  auto upiece = [](int rem) { return PPR == 4 ? (rem >> 2) & 3 : rem % PPR; };
  struct Codes {
    u32x4 w[NP];
    uint32_t sm[NP];
  };
  auto load = [&](Codes& C, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int u = 64 * p + lane;
      const int tsr = u / (16 * PPR), rem = u % (16 * PPR);
      const int row = min(kb * 64 + 16 * wave + urow(rem), R - 1), piece = upiece(rem);
      C.w[p] = __builtin_nontemporal_load(
          (const u32x4*)((tsr ? vc : kc) + (int64_t)row * CB + 16 * piece));
      C.sm[p] = (tsr ? vs_ : ks_)[(int64_t)row * NG + (32 * piece) / 64];
    }
  };
  // A code dword holds dims 0..7 of its piece (low nibble first).  Masking it
  // and its 8-bit shift into the exponents of 1024 and 64 gives the pairs
  // (0, 4), (1, 5), (2, 6), (3, 7) with no byte permute, so every 8-dim
  // chunk of the tiles is stored in that order (Q is loaded in the same
  // order, and the output is put back in flash_store).
  const uint32_t m_lo = in_vgpr(0x64006400u), m_hi = in_vgpr(0x54005400u);
  const f16x2 off_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const f16x2 off_hi = {(_Float16)-64.0f, (_Float16)-64.0f};
  auto expand = [&](const Codes& C, uint8_t* tl) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int u = 64 * p + lane;
      const int tsr = u / (16 * PPR), rem = u % (16 * PPR);
      const int row = 16 * wave + urow(rem), piece = upiece(rem);
      const int swz = swz_k<SPR>(row);
      uint8_t* dst_row = tl + tsr * 64 * RB + row * RB;
      const f16x2 sm = h2_of(C.sm[p]);
      const f16x2 sc = {sm[0], sm[0]}, mn = {sm[1], sm[1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = C.w[p][j], w8 = w >> 8;
        const f16x2 c[4] = {h2_of((w & 0x000F000Fu) | m_lo) + off_lo,
                            h2_of((w & 0x00F000F0u) | m_hi) + off_hi,
                            h2_of((w8 & 0x000F000Fu) | m_lo) + off_lo,
                            h2_of((w8 & 0x00F000F0u) | m_hi) + off_hi};
        u32x4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          y[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c[q], sc, mn));
        *(u32x4*)(dst_row + 16 * ((4 * piece + j) ^ swz)) = y;
      }
    }
  };

  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  auto visible = [&](int kidx) __attribute__((always_inline)) {
    const unsigned t = (unsigned)(kidx - P);
    const bool tree = a.masks ? (bool)((mask >> (t & 63u)) & 1ull) : (int)t <= qi;
    return kidx < R && (kidx < P || tree);
  };
  auto all_visible = [](int) __attribute__((always_inline)) { return true; };
  const int nkb = (R + 63) / 64;
  const int npre = P / 64;  // blocks holding only prefix rows: no per-key test
  Codes C0, C1;
  load(C0, 0);
  load(C1, min(1, nkb - 1));
  expand(C0, tiles);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's tile writes are done
  __builtin_amdgcn_s_barrier();
  // iteration kb: block kb in tiles[kb & 1], block kb + 1's codes in
  // C[(kb + 1) & 1], block kb + 2's codes requested into C[kb & 1].  The
  // expansion is unconditional (past the last block it re-expands that block
  // into the buffer nobody reads), so the expansion and the block step share
  // a basic block and can interleave.
  auto iter = [&](int kb, Codes& Cnext, Codes& Cfree, uint8_t* tcur, uint8_t* tnext, auto vis)
      __attribute__((always_inline)) {
    load(Cfree, min(kb + 2, nkb - 1));
    expand(Cnext, tnext);
    flash_block<D, true>(tcur, tcur + 64 * RB, qf, kb * 64, vis, c2, m_run, l_lane, o);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();  // tnext complete; every wave is done with tcur
  };
  int kb = 0;
  for (; kb + 2 <= npre; kb += 2) {
    iter(kb, C1, C0, tiles, tiles + TILE, all_visible);
    iter(kb + 1, C0, C1, tiles + TILE, tiles, all_visible);
  }
  if (kb < npre) {
    iter(kb, C1, C0, tiles, tiles + TILE, all_visible);
    ++kb;
    // block kb is now in tiles + TILE, its codes' successor in C0
    for (; kb < nkb; kb += 2) {
      iter(kb, C0, C1, tiles + TILE, tiles, visible);
      if (kb + 1 < nkb) iter(kb + 1, C1, C0, tiles, tiles + TILE, visible);
    }
  } else {
    for (; kb < nkb; kb += 2) {
      iter(kb, C1, C0, tiles, tiles + TILE, visible);
      if (kb + 1 < nkb) iter(kb + 1, C0, C1, tiles + TILE, tiles, visible);
    }
  }
  flash_store<D, true>(qi < a.q ? a.out + ((int64_t)r * a.q + qi) * a.h1 + h * D : nullptr, l_lane, o);
}

// -------------------------------------------------------------- launchers
void launch_kv_append(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                      int32_t pos, const int32_t* dpos, const int32_t* rpos, const hp_kv& kv,
                      hipStream_t st) {
  AppendArgs a{(const _Float16*)qkv, b,    q,       h1,     heads,
               h1 / heads,          pos,  dpos,    rpos,   kv.cap,
               kv.k,                kv.v, (uint32_t*)kv.k_sm, (uint32_t*)kv.v_sm,
               kv.page_rows > 0 ? kv.pages : nullptr, kv.page_rows, kv.pool_pages};
  const int64_t tokens = (int64_t)b * q;
  if (tokens == 0) return;
  const int D = h1 / heads;
  if (kv.fmt == HP_Q4 && D == 128 && q >= KT_ROWS && !dpos && !rpos && kv.page_rows == 0 &&
      pos % KT_ROWS == 0 && kv.cap % KT_ROWS == 0) {
    const int64_t grid = (int64_t)b * cdiv(q, KT_ROWS) * cdiv(heads, KT_HEADS);
    Prof prof("kv_append_q4", st);
    hipLaunchKernelGGL(k_kv_append_tile, dim3((unsigned)grid), dim3(256), 0, st, a);
    return;
  }
  const int64_t sc = cdiv(2 * (h1 / 64), 32 * AU);     // workgroups per token
  const int64_t chunks = cdiv(tokens, 16);               // chunks of 16 tokens
  const dim3 grid((unsigned)(8 * cdiv(chunks, 8) * 16 * sc));
  Prof prof(kv.fmt == HP_Q4 ? "kv_append_q4" : "kv_append_f16", st);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a); };
  if (kv.fmt == HP_Q4)
    D == 128 ? go(k_kv_append<true, 128>) : go(k_kv_append<true, 64>);
  else
    D == 128 ? go(k_kv_append<false, 128>) : go(k_kv_append<false, 64>);
}

void launch_decode_attention(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                             int32_t pos, const int32_t* dpos, const int32_t* plen,
                             const uint64_t* masks, const hp_kv& kv, void* out, hipStream_t st) {
  DecArgs a{(const _Float16*)qkv, q,      h1,   heads, pos,  dpos,
            plen,                 masks,  kv.cap, kv.k, kv.v, (const uint32_t*)kv.k_sm,
            (const uint32_t*)kv.v_sm, (_Float16*)out,
            kv.page_rows > 0 ? kv.pages : nullptr, kv.page_rows, kv.pool_pages};
  const int D = h1 / heads;
  if (kv.fmt == HP_Q4 && q >= 16) {
    Prof prof("attn_multi_q4", st);
    const dim3 grid((unsigned)((int64_t)b * heads));
    if (D == 128)
      hipLaunchKernelGGL(k_multi_attn<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_multi_attn<64>, grid, dim3(256), 0, st, a);
    return;
  }
  const dim3 grid((unsigned)((int64_t)b * heads * q));
  Prof prof(kv.fmt == HP_Q4 ? "attn_decode_q4" : "attn_decode_f16", st);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(64), 0, st, a); };
  const bool m = masks != nullptr, q4 = kv.fmt == HP_Q4, paged = a.pages != nullptr;
  auto pick = [&](auto d_, auto q4_) {
    constexpr int Dd = decltype(d_)::value;
    constexpr bool Qq = decltype(q4_)::value;
    if (paged)
      a.cap / a.PR <= 64
          ? (m ? go(k_decode_attn<Dd, Qq, true, 1>) : go(k_decode_attn<Dd, Qq, false, 1>))
          : (m ? go(k_decode_attn<Dd, Qq, true, 2>) : go(k_decode_attn<Dd, Qq, false, 2>));
    else
      m ? go(k_decode_attn<Dd, Qq, true, 0>) : go(k_decode_attn<Dd, Qq, false, 0>);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (D == 128)
    q4 ? pick(I128(), T_()) : pick(I128(), F_());
  else
    q4 ? pick(I64(), T_()) : pick(I64(), F_());
}

void launch_prefill_attention(int32_t b, int32_t s, int32_t h1, int32_t heads, const void* qkv,
                              void* out, hipStream_t st) {
  const int D = h1 / heads;
  const dim3 grid((unsigned)((int64_t)b * heads * cdiv(s, PF_QB)));
  PfArgs a{(const _Float16*)qkv, s, h1, heads, (_Float16*)out};
  Prof prof("attn_prefill", st);
  if (D == 128)
    hipLaunchKernelGGL(k_prefill_attn<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_prefill_attn<64>, grid, dim3(256), 0, st, a);
}

}  // namespace hp
