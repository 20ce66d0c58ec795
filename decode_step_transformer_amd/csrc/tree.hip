// Token trees of speculative decoding ([SpecPipe] article, 2.2.1: token
// index array in BFS order, tree mask M, sub-tree pruning of Fig. 5-b;
// 2.2.2: the tree mask replaces the causal mask and the KV cache keeps the
// verified path, Fig. 8): mask construction, the pruning plan after
// verification, and the move of the kept rows in every layer's cache.
#include "common.h"

namespace hp {

// ------------------------------------------------------------ tree masks
// [SpecPipe] 2.2.1: token i sees itself and its ancestors.  Lane i of a
// wave holds token i of one request.  The ancestor sets come from pointer
// jumping over lane shuffles: after round k, m holds the tokens at distance
// 0 .. 2^k - 1 above token i and a the one at distance 2^k (-1 past the
// root); six rounds cover any depth below 64.  A token whose own parent
// entry breaks the rules (ok false) is treated as a root, so a valid token's
// set stops at, and includes, the first such ancestor.
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t ancestor_set(int i, int q, int p0, bool ok) {
  uint64_t m = i < q ? 1ull << i : 0ull;
  int a = (i < q && ok) ? p0 : -1;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const int from = a < 0 ? i : a;  // every lane takes part in the shuffles
    const uint64_t ma = shfl_u64(m, from);
    const int aa = __shfl(a, from);
    if (a >= 0) {
      m |= ma;
      a = aa;
    }
  }
  return m;
}

__device__ __forceinline__ bool parent_ok(int i, int p) {
  return i == 0 ? p == -1 : (p >= 0 && p < i);
}

// One wave per request (up to 16 waves, each taking every 16th request); an
// entry breaking the parent rules keeps only its own bit and is counted.
__global__ __launch_bounds__(1024) void k_tree_masks(int b, int q, const int32_t* __restrict__ parent,
                                                     uint64_t* __restrict__ masks,
                                                     int32_t* __restrict__ err) {
  __shared__ int bad[16];
  const int i = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int nbad = 0;
  for (int r = w; r < b; r += nw) {
    const int p0 = i < q ? parent[(int64_t)r * q + i] : -1;
    const bool ok = i >= q || parent_ok(i, p0);
    nbad += ok ? 0 : 1;
    const uint64_t m = ancestor_set(i, q, p0, ok);
    if (i < q) masks[(int64_t)r * q + i] = m;
  }
  for (int o = 32; o > 0; o >>= 1) nbad += __shfl_xor(nbad, o);
  if (i == 0) bad[w] = nbad;
  __syncthreads();
  if (threadIdx.x == 0 && err) {
    int t = 0;
    for (int j = 0; j < nw; ++j) t += bad[j];
    *err = t;
  }
}

// ------------------------------------------------------------ tree pruning
// [SpecPipe] 2.2.1 sub-tree pruning (Fig. 5-b) and 2.2.2 (Fig. 8): once
// token u of a request is verified, column u of the mask matrix (u and its
// descendants) is the new tree, with u as its root; the verified path above
// u (row u of the mask without u) stays in the cache as committed prefix.
// One wave per request; lane i holds token i: its ancestor set as in
// k_tree_masks, u's set broadcast by a shuffle.  The rows that stay in the
// cache (path, then subtree) are the lanes flagged in either set, in index
// order: a ballot prefix count gives each its position, and the subtree
// tokens' positions less the path length are their new indices; a shuffle
// maps each parent to its new index.  Slots past the new tree are filler
// leaves (the last kept token's parent, or 0 when u is alone) so the new
// array stays a valid BFS parent array.  A request with an invalid parent
// array or verified index keeps nothing and is counted in err.
__global__ __launch_bounds__(1024) void k_tree_prune(int b, int q, int pos,
                                                     const int32_t* __restrict__ parent,
                                                     const int32_t* __restrict__ verified,
                                                     int32_t* __restrict__ new_parent,
                                                     int32_t* __restrict__ src,
                                                     int32_t* __restrict__ prefix_out,
                                                     int32_t* __restrict__ kept_out,
                                                     int32_t* __restrict__ err) {
  __shared__ int bad[16];
  const int i = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int nbad = 0;
  for (int r = w; r < b; r += nw) {
    const int p0 = i < q ? parent[(int64_t)r * q + i] : -1;
    const bool ok = i >= q || parent_ok(i, p0);
    const int u = verified[r];
    const bool good = !__any(!ok) && u >= 0 && u < q;
    int32_t* npr = new_parent + (int64_t)r * q;
    int32_t* sr = src + (int64_t)r * q;
    if (!good) {
      if (i == 0) {
        kept_out[r] = 0;
        prefix_out[r] = pos;
        ++nbad;
      }
      if (i < q) {
        npr[i] = i == 0 ? -1 : 0;
        sr[i] = -1;
      }
      continue;
    }
    const uint64_t m = ancestor_set(i, q, p0, true);
    const uint64_t mu = shfl_u64(m, u);
    const int depth = __popcll(mu) - 1;                  // u's ancestors
    const bool in_sub = i < q && ((m >> u) & 1ull);      // u or below it
    const bool stay = in_sub || (i < q && ((mu >> i) & 1ull));
    const uint64_t sb = __ballot(stay);
    const int row = __popcll(sb & ((1ull << i) - 1ull));  // position after the old prefix
    const int rows = __popcll(sb);
    const int kept = rows - depth;
    const int nidx = row - depth;                          // new index (subtree lanes)
    const int nidx_of_parent = __shfl(nidx, p0 < 0 ? 0 : p0);
    const int np = (i == u || p0 < 0) ? -1 : nidx_of_parent;
    const int last = 63 - __clzll(sb);  // lane of the last kept token (in the subtree)
    const int np_last = __shfl(np, last);
    const int fill = kept == 1 ? 0 : np_last;
    if (stay) sr[row] = i;
    if (i < q && i >= rows) sr[i] = -1;
    if (in_sub) npr[nidx] = np;
    if (i < q && i >= kept) npr[i] = fill;
    if (i == 0) {
      kept_out[r] = kept;
      prefix_out[r] = pos + depth;
    }
  }
  if (i == 0) bad[w] = nbad;
  __syncthreads();
  if (threadIdx.x == 0 && err) {
    int t = 0;
    for (int j = 0; j < nw; ++j) t += bad[j];
    *err = t;
  }
}

// Moves the rows that stay after k_tree_prune into place: one wave per
// (request, head, K or V); lane j (j < prefix - pos + kept: the committed
// path, then the new tree) copies cache row pos + src[j] to row pos + j (RB
// bytes of codes or fp16, SMB bytes of scale/min pairs).  Every lane's store
// depends on its own load and each load instruction covers the whole wave,
// so all rows are read before any is overwritten.
template <int RB, int SMB>
__global__ __launch_bounds__(64) void k_kv_compact(int q, int heads, int pos, int cap,
                                                   const int32_t* __restrict__ src,
                                                   const int32_t* __restrict__ prefix,
                                                   const int32_t* __restrict__ kept, uint8_t* k,
                                                   uint8_t* v, uint8_t* ksm, uint8_t* vsm) {
  const int j = threadIdx.x;
  const int t = blockIdx.x & 1, rh = blockIdx.x >> 1;
  const int h = rh % heads, r = rh / heads;
  // any prefix / kept / src values keep the moves inside rows [pos, pos + q)
  const int n = min(max(prefix[r] - pos + kept[r], 0), q);
  const int64_t row0 = (int64_t)(r * heads + h) * cap + pos;
  uint8_t* base = (t ? v : k) + row0 * RB;
  uint8_t* sbase = SMB ? (t ? vsm : ksm) + row0 * SMB : nullptr;
  const int s = j < n ? src[(int64_t)r * q + j] : j;
  const bool act = j < n && s >= 0 && s < q;
  u32x4 buf[RB / 16];
  uint32_t sm[SMB / 4 > 0 ? SMB / 4 : 1];
  if (act) {
#pragma unroll
    for (int c = 0; c < RB / 16; ++c) buf[c] = *(const u32x4*)(base + (int64_t)s * RB + 16 * c);
#pragma unroll
    for (int c = 0; c < SMB / 4; ++c) sm[c] = *(const uint32_t*)(sbase + (int64_t)s * SMB + 4 * c);
  }
  if (act && s != j) {
#pragma unroll
    for (int c = 0; c < RB / 16; ++c) *(u32x4*)(base + (int64_t)j * RB + 16 * c) = buf[c];
#pragma unroll
    for (int c = 0; c < SMB / 4; ++c) *(uint32_t*)(sbase + (int64_t)j * SMB + 4 * c) = sm[c];
  }
}

// -------------------------------------------------------------- launchers
void launch_tree_masks(int32_t b, int32_t q, const int32_t* parent, uint64_t* masks, int32_t* err,
                       hipStream_t st) {
  Prof prof("tree_masks", st);
  hipLaunchKernelGGL(k_tree_masks, dim3(1), dim3(64 * std::min(b, 16)), 0, st, b, q, parent,
                     masks, err);
}

void launch_tree_prune(int32_t b, int32_t q, int32_t pos, const int32_t* parent,
                       const int32_t* verified, int32_t* new_parent, int32_t* src,
                       int32_t* prefix, int32_t* kept, int32_t* err, hipStream_t st) {
  Prof prof("tree_prune", st);
  hipLaunchKernelGGL(k_tree_prune, dim3(1), dim3(64 * std::min(b, 16)), 0, st, b, q, pos, parent,
                     verified, new_parent, src, prefix, kept, err);
}

void launch_kv_compact(int32_t b, int32_t q, int32_t heads, int32_t d, int32_t pos,
                       const int32_t* src, const int32_t* prefix, const int32_t* kept,
                       const hp_kv& kv, hipStream_t st) {
  const dim3 grid((unsigned)(2 * b * heads));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(64), 0, st, q, heads, pos, kv.cap, src, prefix, kept,
                       (uint8_t*)kv.k, (uint8_t*)kv.v, (uint8_t*)kv.k_sm, (uint8_t*)kv.v_sm);
  };
  Prof prof("kv_compact", st);
  if (kv.fmt == HP_Q4) {
    if (d == 128)
      go(k_kv_compact<64, 8>);
    else
      go(k_kv_compact<32, 4>);
  } else {
    if (d == 128)
      go(k_kv_compact<256, 0>);
    else
      go(k_kv_compact<128, 0>);
  }
}

}  // namespace hp
