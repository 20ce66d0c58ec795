// KV-cache append and attention for the FlexGen layer ([FlexGen] paper
// notes, background section: prefill and decode equations; section 5: the KV
// cache is stored as int4 groups of 64 along the hidden dimension and
// converted back before use; [SpecPipe] 2.2.1-2.2.2: tree masks).
//
// Decode attention is HBM-bound (about 1 flop per byte of packed cache), so
// it runs on the vector ALUs, one wave per (request, head, query):
//  * score phase: lane = cache row; the lane streams its row's 64 bytes of
//    codes with 16-byte loads and forms the dot product with packed
//    fp16 dot2 on exact small-integer halves, factoring the group scale and
//    min out of the sum: s = sum_g scale_g * (q . c)_g + min_g * (sum q)_g;
//  * online softmax across 64-row chunks with wave reductions;
//  * value phase: 16 lanes cover one row (one dword = 8 codes each), 4 rows
//    at a time; sum_t p_t v_t = sum_t (p_t scale_t) c_t + sum_t p_t min_t,
//    the second term accumulated per group in the score phase.
// Prefill attention reads the fresh fp16 K/V of the prompt (causal), one wave
// per (request, head, 64 queries), lane = query, key tiles staged in LDS.
#include <math.h>

#include "common.h"
#include "quant_dev.h"

namespace hp {

// ------------------------------------------------------------ KV append
struct AppendArgs {
  const _Float16* qkv;
  int b, q, h1, H, D, pos;
  const int32_t* dpos;
  int cap;
  void* k;
  void* v;
  uint32_t* ksm;
  uint32_t* vsm;
};

template <bool Q4>
__global__ __launch_bounds__(256) void k_kv_append(AppendArgs a) {
  const int sub = threadIdx.x & 7;
  const int G = a.D / 64;
  const int64_t groups = 2LL * a.b * a.q * a.H * G;
  const int pos = a.pos + (a.dpos ? *a.dpos : 0);
  const int64_t stride = (int64_t)gridDim.x * 32;
  for (int64_t gi = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); gi < groups; gi += stride) {
    int64_t rest = gi;
    const int g = (int)(rest % G);
    rest /= G;
    const int h = (int)(rest % a.H);
    rest /= a.H;
    const int i = (int)(rest % a.q);
    rest /= a.q;
    const int r = (int)(rest % a.b);
    const int which = (int)(rest / a.b);  // 0 = K, 1 = V
    const _Float16* src =
        a.qkv + ((int64_t)r * a.q + i) * 3 * a.h1 + (int64_t)(1 + which) * a.h1 + h * a.D + 64 * g;
    const uint4 raw = *(const uint4*)(src + 8 * sub);
    const int64_t row = ((int64_t)r * a.H + h) * a.cap + pos + i;
    if constexpr (Q4) {
      uint32_t smw;
      const uint32_t word = quant_group8(raw, smw);
      uint8_t* dst = (uint8_t*)(which ? a.v : a.k) + row * (a.D / 2) + 32 * g;
      *(uint32_t*)(dst + 4 * sub) = word;
      if (sub == 0) (which ? a.vsm : a.ksm)[row * G + g] = smw;
    } else {
      _Float16* dst = (_Float16*)(which ? a.v : a.k) + row * a.D + 64 * g;
      *(uint4*)(dst + 8 * sub) = raw;
    }
  }
}

// ------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ f16x2 h2_of(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// ------------------------------------------------------- decode attention
struct DecArgs {
  const _Float16* qkv;
  int q, h1, H, pos;
  const int32_t* dpos;
  const uint64_t* masks;
  int cap;
  const void* k;
  const void* v;
  const uint32_t* ksm;
  const uint32_t* vsm;
  _Float16* out;
};

template <int D, bool Q4>
__global__ __launch_bounds__(64) void k_decode_attn(DecArgs a) {
  constexpr int G = D / 64;            // int4 groups per row
  constexpr int SEGS = D / 8;          // lanes per row in the value phase
  constexpr int RSUB = 64 / SEGS;      // rows per value-phase step
  __shared__ float ps[64][G];          // p_t * scale_{t,g} (Q4) or p_t (F16, g = 0)

  const int lane = threadIdx.x;
  const int i = blockIdx.x % a.q;
  const int rh = blockIdx.x / a.q;
  const int h = rh % a.H, r = rh / a.H;
  const int P = a.pos + (a.dpos ? *a.dpos : 0);
  const int R = a.masks ? P + a.q : P + i + 1;
  const uint64_t mask = a.masks ? a.masks[(int64_t)r * a.q + i] : 0ull;
  const int64_t rowbase = ((int64_t)r * a.H + h) * a.cap;
  const float scale = 1.0f / sqrtf((float)D);

  // query as binary16 pairs, in the pairing order of the score phase
  f16x2 q2[D / 2];
  float qsum[G];
  {
    const uint4* qp = (const uint4*)(a.qkv + ((int64_t)r * a.q + i) * 3 * a.h1 + h * D);
#pragma unroll
    for (int g = 0; g < G; ++g) qsum[g] = 0.f;
#pragma unroll
    for (int w = 0; w < D / 8; ++w) {
      const uint4 raw = qp[w];
      const f16x8 qh = __builtin_bit_cast(f16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) qsum[(8 * w) / 64] += (float)qh[e];
      if constexpr (Q4) {
#pragma unroll
        for (int p = 0; p < 4; ++p) q2[4 * w + p] = f16x2{qh[p], qh[p + 4]};
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) q2[4 * w + p] = f16x2{qh[2 * p], qh[2 * p + 1]};
      }
    }
  }

  const int rsub = lane / SEGS, seg = lane % SEGS;
  const int gl = (8 * seg) / 64;       // group of this lane's value dims
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float pm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) pm[g] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const f16x2 off1024 = {(_Float16)1024.0f, (_Float16)1024.0f};

  for (int base = 0; base < R; base += 64) {
    const int row = base + lane;
    const bool valid =
        row < R && (!a.masks || row < P || ((mask >> (unsigned)(row - P)) & 1ull));
    float s = -INFINITY;
    float vs[G], vm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) vs[g] = vm[g] = 0.f;
    if (valid) {
      if constexpr (Q4) {
        const uint4* kp = (const uint4*)((const uint8_t*)a.k + (rowbase + row) * (D / 2));
        uint4 kc[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kc[c] = kp[c];
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const uint32_t ws[4] = {kc[c].x, kc[c].y, kc[c].z, kc[c].w};
#pragma unroll
          for (int wj = 0; wj < 4; ++wj) {
            const int w = 4 * c + wj;  // dword index within the row: elements 8w .. 8w+7
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t u = ((ws[wj] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
              const f16x2 cc = h2_of(u) - off1024;
              dot[(8 * w) / 64] = __builtin_amdgcn_fdot2(cc, q2[4 * w + p], dot[(8 * w) / 64], false);
            }
          }
        }
        s = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t ksm = a.ksm[(rowbase + row) * G + g];
          const float sc = (float)h2_of(ksm)[0], mn = (float)h2_of(ksm)[1];
          s += sc * dot[g] + mn * qsum[g];
          const uint32_t vsm = a.vsm[(rowbase + row) * G + g];
          vs[g] = (float)h2_of(vsm)[0];
          vm[g] = (float)h2_of(vsm)[1];
        }
      } else {
        const uint4* kp = (const uint4*)((const _Float16*)a.k + (rowbase + row) * D);
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          const uint4 kv = kp[c];
          const uint32_t ws[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) dot = __builtin_amdgcn_fdot2(h2_of(ws[p]), q2[4 * c + p], dot, false);
        }
        s = dot;
      }
      s *= scale;
    }
    const float cmax = wave_max(s);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    const float p = valid ? expf(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    if constexpr (Q4) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pm[g] = pm[g] * alpha + p * vm[g];
        ps[lane][g] = p * vs[g];
      }
    } else {
      ps[lane][0] = p;
    }
    __syncthreads();
    const int rows = min(64, R - base);
    for (int t = rsub; t < rows; t += RSUB) {
      const int64_t vrow = rowbase + base + t;
      if constexpr (Q4) {
        const uint32_t w = *(const uint32_t*)((const uint8_t*)a.v + vrow * (D / 2) + 4 * seg);
        const float pw = ps[t][gl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += pw * (float)((w >> (4 * e)) & 15u);
      } else {
        const uint4 vv = *(const uint4*)((const _Float16*)a.v + vrow * D + 8 * seg);
        const f16x8 vh = __builtin_bit_cast(f16x8, vv);
        const float pw = ps[t][0];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += pw * (float)vh[e];
      }
    }
    __syncthreads();
  }

  // combine the RSUB row groups, then the per-group min term
#pragma unroll
  for (int off = SEGS; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  float pmg = 0.f;
  if constexpr (Q4) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float t = wave_sum(pm[g]);
      if (g == gl) pmg = t;
    }
  }
  if (rsub == 0) {
    const float inv = 1.0f / l_run;
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)((acc[e] + pmg) * inv);
    *(f16x8*)(a.out + ((int64_t)r * a.q + i) * a.h1 + h * D + 8 * seg) = o;
  }
}

// ------------------------------------------------------ prefill attention
// Causal attention over the fresh K/V of the prompt: query i sees keys 0..i.
constexpr int PF_KT = 16;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(64) void k_prefill_attn(const _Float16* __restrict__ qkv, int s,
                                                     int h1, int H, _Float16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 Ks[PF_KT][D];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[PF_KT][D];
  const int lane = threadIdx.x;
  const int nqb = (s + 63) / 64;
  const int qb = blockIdx.x % nqb;
  const int rh = blockIdx.x / nqb;
  const int h = rh % H, r = rh / H;
  const int qi = qb * 64 + lane;
  const bool qv = qi < s;
  const int64_t ld = 3LL * h1;
  const _Float16* base = qkv + (int64_t)r * s * ld + h * D;
  const float scale = 1.0f / sqrtf((float)D);

  f16x2 q2[D / 2];
  {
    const uint4* qp = (const uint4*)(base + (int64_t)(qv ? qi : 0) * ld);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 raw = qp[c];
      q2[4 * c + 0] = h2_of(raw.x);
      q2[4 * c + 1] = h2_of(raw.y);
      q2[4 * c + 2] = h2_of(raw.z);
      q2[4 * c + 3] = h2_of(raw.w);
    }
  }
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int kend = min(s, qb * 64 + 64);
  for (int k0 = 0; k0 < kend; k0 += PF_KT) {
    __syncthreads();
    // stage PF_KT rows of K and V: PF_KT * D / 8 16-byte chunks each
    for (int c = lane; c < PF_KT * D / 8; c += 64) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (k0 + row < s) {
        kv = *(const uint4*)(base + (int64_t)(k0 + row) * ld + h1 + col);
        vv = *(const uint4*)(base + (int64_t)(k0 + row) * ld + 2 * h1 + col);
      }
      *(uint4*)&Ks[row][col] = kv;
      *(uint4*)&Vs[row][col] = vv;
    }
    __syncthreads();
    float sc[PF_KT];
    float cmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < PF_KT; ++j) {
      const int kj = k0 + j;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const uint4 kv = *(const uint4*)&Ks[j][8 * c];
        dot = __builtin_amdgcn_fdot2(h2_of(kv.x), q2[4 * c + 0], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_of(kv.y), q2[4 * c + 1], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_of(kv.z), q2[4 * c + 2], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_of(kv.w), q2[4 * c + 3], dot, false);
      }
      sc[j] = (kj <= qi && kj < s) ? dot * scale : -INFINITY;
      cmax = fmaxf(cmax, sc[j]);
    }
    const float m_new = fmaxf(m_run, cmax);
    if (m_new == -INFINITY) continue;  // no visible key yet for this lane
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < PF_KT; ++j) {
      sc[j] = (sc[j] == -INFINITY) ? 0.f : expf(sc[j] - m_new);
      psum += sc[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      float a8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] = acc[c + e] * alpha;
#pragma unroll
      for (int j = 0; j < PF_KT; ++j) {
        const f16x8 vh = *(const f16x8*)&Vs[j][c];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] += sc[j] * (float)vh[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c + e] = a8[e];
    }
  }
  if (!qv) return;
  const float inv = 1.0f / l_run;
  _Float16* o = out + ((int64_t)r * s + qi) * h1 + h * D;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    f16x8 v8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v8[e] = (_Float16)(acc[c + e] * inv);
    *(f16x8*)(o + c) = v8;
  }
}

// ------------------------------------------------------------ tree masks
// [SpecPipe] 2.2.1: token i sees itself and its ancestors.  One workgroup
// walks every request; an entry breaking the parent rules keeps only its own
// bit and is counted.
__global__ __launch_bounds__(64) void k_tree_masks(int b, int q, const int32_t* __restrict__ parent,
                                                   uint64_t* __restrict__ masks,
                                                   int32_t* __restrict__ err) {
  __shared__ int bad[64];
  const int i = threadIdx.x;
  int nbad = 0;
  for (int r = 0; r < b; ++r) {
    if (i < q) {
      const int32_t* pr = parent + (int64_t)r * q;
      const int p0 = pr[i];
      const bool ok = (i == 0) ? (p0 == -1) : (p0 >= 0 && p0 < i);
      nbad += ok ? 0 : 1;
      uint64_t m = 1ull << i;
      if (ok) {
        int u = p0;
        while (u >= 0) {  // parents strictly decrease along valid links
          m |= 1ull << u;
          const int pu = pr[u];
          if (!(u == 0 ? pu == -1 : (pu >= 0 && pu < u))) break;
          u = pu;
        }
      }
      masks[(int64_t)r * q + i] = m;
    }
  }
  bad[i] = nbad;
  __syncthreads();
  if (i == 0) {
    int t = 0;
    for (int j = 0; j < 64; ++j) t += bad[j];
    if (err) *err = t;
  }
}

// -------------------------------------------------------------- launchers
void launch_kv_append(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                      int32_t pos, const int32_t* dpos, const hp_kv& kv, hipStream_t st) {
  AppendArgs a{(const _Float16*)qkv, b,  q,        h1,   heads,
               h1 / heads,          pos, dpos,     kv.cap, kv.k,
               kv.v,                (uint32_t*)kv.k_sm, (uint32_t*)kv.v_sm};
  const int64_t groups = 2LL * b * q * heads * ((h1 / heads) / 64);
  if (groups == 0) return;
  const int blocks = (int)std::min<int64_t>(cdiv(groups, 32), 16384);
  Prof prof(kv.fmt == HP_Q4 ? "kv_append_q4" : "kv_append_f16", st);
  if (kv.fmt == HP_Q4)
    hipLaunchKernelGGL(k_kv_append<true>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_kv_append<false>, dim3(blocks), dim3(256), 0, st, a);
}

void launch_decode_attention(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                             int32_t pos, const int32_t* dpos, const uint64_t* masks,
                             const hp_kv& kv, void* out, hipStream_t st) {
  DecArgs a{(const _Float16*)qkv, q,     h1,   heads, pos,  dpos,
            masks,                kv.cap, kv.k, kv.v,  (const uint32_t*)kv.k_sm,
            (const uint32_t*)kv.v_sm, (_Float16*)out};
  const int D = h1 / heads;
  const dim3 grid((unsigned)((int64_t)b * heads * q));
  Prof prof(kv.fmt == HP_Q4 ? "attn_decode_q4" : "attn_decode_f16", st);
  if (D == 128) {
    if (kv.fmt == HP_Q4)
      hipLaunchKernelGGL((k_decode_attn<128, true>), grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_attn<128, false>), grid, dim3(64), 0, st, a);
  } else {
    if (kv.fmt == HP_Q4)
      hipLaunchKernelGGL((k_decode_attn<64, true>), grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_attn<64, false>), grid, dim3(64), 0, st, a);
  }
}

void launch_prefill_attention(int32_t b, int32_t s, int32_t h1, int32_t heads, const void* qkv,
                              void* out, hipStream_t st) {
  const int D = h1 / heads;
  const dim3 grid((unsigned)((int64_t)b * heads * cdiv(s, 64)));
  Prof prof("attn_prefill", st);
  if (D == 128)
    hipLaunchKernelGGL(k_prefill_attn<128>, grid, dim3(64), 0, st, (const _Float16*)qkv, s, h1,
                       heads, (_Float16*)out);
  else
    hipLaunchKernelGGL(k_prefill_attn<64>, grid, dim3(64), 0, st, (const _Float16*)qkv, s, h1,
                       heads, (_Float16*)out);
}

void launch_tree_masks(int32_t b, int32_t q, const int32_t* parent, uint64_t* masks, int32_t* err,
                       hipStream_t st) {
  Prof prof("tree_masks", st);
  hipLaunchKernelGGL(k_tree_masks, dim3(1), dim3(64), 0, st, b, q, parent, masks, err);
}

}  // namespace hp
