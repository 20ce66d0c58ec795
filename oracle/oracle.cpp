// CPU oracle for the FlexGen OPT-style layer with group-wise int4 compression.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline leg of the benchmark may load this library.  It shares no code,
// header, table or helper with the HIP library: every definition here is
// written out again from the pages.
//
// Sources (page titles as cited throughout):
//   [FlexGen]  "FlexGen: High-Throughput Generative Inference of Large Language
//              Models with a Single GPU" (paper notes, ICML 2023).
//   [SpecPipe] "大语言模型推理加速：SpecPipe技术解析与实践" (article).
//
// Arithmetic: sums (matrix products, attention scores and weighted sums,
// softmax) run in double precision with a fixed ascending order; values are
// rounded to IEEE binary16 exactly where the pages store FP16 tensors.  The
// quantiser's integer decision is taken in binary32, the precision the GPU
// kernel takes it in, with the same IEEE operations (see or_quantize_g64).
//
// Layouts (all row-major, binary16 passed as raw uint16 bits):
//   matrix w, page orientation x·w:  w[h_in][h_out]
//   activations:                     x[rows][h1], rows = requests x tokens
//   KV cache, fp16 format:           k[b][heads][cap][d]
//   KV cache, int4 group-64 format:  codes[b][heads][cap][d/2] (byte j holds
//                                    codes 2j | 2j+1 << 4), and
//                                    sm[b][heads][cap][d/64][2] = {scale, min}
//   group-64 tensor (any):           codes[rows][cols/2], sm[rows][cols/64][2]
//
// Parity pins: tests/test_oracle_*.py check every function here against values
// and identities fixed by the pages and by mathematics (see each function).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <omp.h>

typedef int64_t i64;

extern "C" {

// ---------------------------------------------------------------- binary16
// IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
float or_h2f(uint16_t h) {
  const int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  float v;
  if (e == 0)
    v = std::ldexp((float)f, -24);  // zero or subnormal
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = std::ldexp((float)(f | 1024), e - 25);
  return sign ? -v : v;
}

// Round a double to the nearest binary16, ties to even, with subnormals; a
// magnitude of 65520 or more (half an ulp above 65504) becomes infinity.
uint16_t or_d2h(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  if (std::isnan(x)) return sign | 0x7e00;
  double a = std::fabs(x);
  if (a >= 65520.0) return sign | 0x7c00;
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);                      // a in [2^(e2-1), 2^e2)
  const int E = e2 - 1;                    // unbiased exponent of a
  const int qexp = (E < -14) ? -24 : E - 10;  // weight of the last kept bit
  const double n = std::nearbyint(std::ldexp(a, -qexp));  // RNE to an integer
  const double v = std::ldexp(n, qexp);    // the rounded magnitude, exact
  if (v == 0.0) return sign;
  if (v < std::ldexp(1.0, -14))            // subnormal: fraction = v / 2^-24
    return sign | (uint16_t)std::ldexp(v, 24);
  int ev;
  std::frexp(v, &ev);
  const int Ev = ev - 1;
  const uint16_t frac = (uint16_t)(std::ldexp(v, 10 - Ev) - 1024.0);
  return sign | (uint16_t)((Ev + 15) << 10) | frac;
}

uint16_t or_f2h(float x) { return or_d2h((double)x); }

void or_h2f_array(const uint16_t* h, float* f, i64 n) {
  for (i64 i = 0; i < n; ++i) f[i] = or_h2f(h[i]);
}
void or_f2h_array(const float* f, uint16_t* h, i64 n) {
  for (i64 i = 0; i < n; ++i) h[i] = or_f2h(f[i]);
}
void or_d2h_array(const double* d, uint16_t* h, i64 n) {
  for (i64 i = 0; i < n; ++i) h[i] = or_d2h(d[i]);
}

int or_threads(void) { return omp_get_max_threads(); }

// ------------------------------------------------- group-wise int4 quantiser
// [FlexGen] section 5 (group-wise quantization, eq. for x_quant): a group is
// g = 64 consecutive elements along one dimension; each element becomes
// round((x - min) / (max - min) * (2^b - 1)) with b = 4.  Readings where the
// page is silent:
//  * the quotient is evaluated in binary32 in the printed order,
//    ((x - min) / (max - min)) * 15, each operation correctly rounded;
//  * round() is round-half-to-even (IEEE rint);
//  * -0 counts as +0; NaN elements are skipped by min/max and get code 0;
//  * a group whose max - min is not > 0 gets codes 0 and scale 0;
//  * stored per group: scale = fp16((max - min) / 15), min = fp16(min)
//    (exact, since min is one of the fp16 elements).
static void quant_group(const uint16_t* x, uint8_t* codes, uint16_t* sm) {
  float xs[64];
  float mn = INFINITY, mx = -INFINITY;
  for (int i = 0; i < 64; ++i) {
    xs[i] = or_h2f(x[i]) + 0.0f;
    mn = std::fmin(mn, xs[i]);
    mx = std::fmax(mx, xs[i]);
  }
  const float r = mx - mn;
  uint8_t c[64];
  if (!(r > 0.0f)) {
    for (int i = 0; i < 64; ++i) c[i] = 0;
    sm[0] = 0;
    sm[1] = std::isfinite(mn) ? or_f2h(mn) : 0;
  } else {
    sm[0] = or_f2h(r / 15.0f);
    sm[1] = or_f2h(mn);
    for (int i = 0; i < 64; ++i) {
      const float t = (xs[i] - mn) / r * 15.0f;
      float q = std::rint(t);
      q = std::fmin(std::fmax(q, 0.0f), 15.0f);
      c[i] = (uint8_t)q;
    }
  }
  for (int j = 0; j < 32; ++j) codes[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
}

// Groups run along the contiguous dimension: x[rows][cols], cols % 64 == 0.
void or_quantize_g64(const uint16_t* x, i64 rows, i64 cols, uint8_t* codes, uint16_t* sm) {
  const i64 ng = cols / 64;
#pragma omp parallel for schedule(static)
  for (i64 r = 0; r < rows; ++r)
    for (i64 g = 0; g < ng; ++g)
      quant_group(x + r * cols + g * 64, codes + r * (cols / 2) + g * 32, sm + (r * ng + g) * 2);
}

// [FlexGen] section 5: stored tensors are converted back to FP16 before any
// computation.  Reading: y = fp16(c * scale + min) with one rounding (the
// product and sum are exact in double).
static inline uint16_t dequant_one(int c, uint16_t scale, uint16_t mn) {
  return or_d2h((double)c * (double)or_h2f(scale) + (double)or_h2f(mn));
}

void or_dequantize_g64(const uint8_t* codes, const uint16_t* sm, i64 rows, i64 cols, uint16_t* y) {
  const i64 ng = cols / 64;
#pragma omp parallel for schedule(static)
  for (i64 r = 0; r < rows; ++r)
    for (i64 i = 0; i < cols; ++i) {
      const uint8_t byte = codes[r * (cols / 2) + i / 2];
      const int c = (i & 1) ? (byte >> 4) : (byte & 15);
      const uint16_t* s = sm + (r * ng + i / 64) * 2;
      y[r * cols + i] = dequant_one(c, s[0], s[1]);
    }
}

// ------------------------------------------------------------ matrix product
// [FlexGen] background section, prefill and decode equations: every
// projection is a product x·w with w[h_in][h_out].  y[m][n] =
// fp16( act( sum_k x[m][k] w[k][n] ) + res[m][n] ), summed over k in ascending
// order in double; act is relu or identity; res may be absent.
void or_gemm(const uint16_t* x, i64 ldx, const uint16_t* w, i64 M, i64 K, i64 N,
             const uint16_t* res, i64 ldr, int relu, uint16_t* y, i64 ldy) {
  // Work is split over blocks of 256 output columns (each block takes all M
  // rows); every output still sums its K products in ascending k.
  const i64 NB = 256, nblk = (N + NB - 1) / NB;
#pragma omp parallel for schedule(dynamic, 1)
  for (i64 blk = 0; blk < nblk; ++blk) {
    const i64 n0 = blk * NB, nn = std::min(NB, N - n0);
    std::vector<double> acc((size_t)(M * nn), 0.0), wk((size_t)nn);
    for (i64 k = 0; k < K; ++k) {
      for (i64 n = 0; n < nn; ++n) wk[(size_t)n] = or_h2f(w[k * N + n0 + n]);
      for (i64 m = 0; m < M; ++m) {
        const double a = or_h2f(x[m * ldx + k]);
        double* am = acc.data() + (size_t)(m * nn);
        for (i64 n = 0; n < nn; ++n) am[n] += a * wk[(size_t)n];
      }
    }
    for (i64 m = 0; m < M; ++m)
      for (i64 n = 0; n < nn; ++n) {
        double v = acc[(size_t)(m * nn + n)];
        if (relu) v = v > 0.0 ? v : 0.0;
        if (res) v += or_h2f(res[m * ldr + n0 + n]);
        y[m * ldy + n0 + n] = or_d2h(v);
      }
  }
}

// ---------------------------------------------------------------- attention
// [FlexGen] background section: softmax(q k^T / sqrt(.)) v per query row.
// Reading for several heads: head h uses channels [h d, (h+1) d) of q, k, v,
// with d = h1 / heads and the scale 1/sqrt(d) (one head gives the page's
// 1/sqrt(h1)).  Query i sees the keys j < lim[i], plus key tbase + u for
// every bit u set in mask[i] (mask may be null).  Keys and values are fp16
// values; the result is rounded to fp16.  Scores, exponentials and sums are
// double; the softmax subtracts the row maximum first.
static void attn_rows(int d, int nq, const uint16_t* q, i64 ldq, const uint16_t* k,
                      const uint16_t* v, i64 ldkv, const int* lim, const uint64_t* mask,
                      int tbase, uint16_t* out, i64 ldo) {
  const double scale = 1.0 / std::sqrt((double)d);
  std::vector<int> vis;
  std::vector<double> z, acc((size_t)d);
  for (int i = 0; i < nq; ++i) {
    vis.clear();
    for (int j = 0; j < lim[i]; ++j) vis.push_back(j);
    if (mask)
      for (int u = 0; u < 64; ++u)
        if ((mask[i] >> u) & 1ull) vis.push_back(tbase + u);
    z.assign(vis.size(), 0.0);
    double mx = -INFINITY;
    for (size_t t = 0; t < vis.size(); ++t) {
      const i64 j = vis[t];
      double s = 0.0;
      for (int c = 0; c < d; ++c) s += (double)or_h2f(q[i * ldq + c]) * (double)or_h2f(k[j * ldkv + c]);
      z[t] = s * scale;
      if (z[t] > mx) mx = z[t];
    }
    double den = 0.0;
    for (size_t t = 0; t < vis.size(); ++t) {
      z[t] = std::exp(z[t] - mx);
      den += z[t];
    }
    for (int c = 0; c < d; ++c) acc[(size_t)c] = 0.0;
    for (size_t t = 0; t < vis.size(); ++t) {
      const i64 j = vis[t];
      for (int c = 0; c < d; ++c) acc[(size_t)c] += z[t] * (double)or_h2f(v[j * ldkv + c]);
    }
    for (int c = 0; c < d; ++c) out[i * ldo + c] = or_d2h(acc[(size_t)c] / den);
  }
}

// Plain attention entry for tests: q[nq][d], k and v [T][d]; visibility as above.
void or_attention(int d, int nq, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const int* lim, const uint64_t* mask, int tbase, uint16_t* out) {
  attn_rows(d, nq, q, d, k, v, d, lim, mask, tbase, out, d);
}

// ------------------------------------------------------------- KV cache I/O
// [FlexGen] section 5: the KV cache is stored compressed, groups of 64 along
// the hidden dimension; [FlexGen] decode equations: new rows are
// concatenated.  Format 0: fp16 rows k[b][H][cap][d].  Format 1: int4
// group-64 rows codes[b][H][cap][d/2] and sm[b][H][cap][d/64][2].
enum { OR_F16 = 0, OR_Q4 = 1 };

// Write token rows src (one request: src[qi][h1], row stride ld) into rows
// [pos, pos + nq) of request r's cache.
static void kv_store(int fmt, int H, int d, int cap, int r, int pos, int nq, const uint16_t* src,
                     i64 ld, void* store, uint16_t* sm) {
  for (int h = 0; h < H; ++h)
    for (int i = 0; i < nq; ++i) {
      const i64 row = ((i64)r * H + h) * cap + pos + i;
      const uint16_t* s = src + (i64)i * ld + (i64)h * d;
      if (fmt == OR_F16) {
        std::memcpy((uint16_t*)store + row * d, s, sizeof(uint16_t) * d);
      } else {
        for (int g = 0; g < d / 64; ++g)
          quant_group(s + 64 * g, (uint8_t*)store + row * (d / 2) + 32 * g,
                      sm + (row * (d / 64) + g) * 2);
      }
    }
}

// Concat of given K/V token rows into the cache ([FlexGen] background
// section, decode: the new k and v rows are concatenated to the cache; section
// 5: stored as int4 groups of 64 along the hidden dimension): k_rows and
// v_rows are [b][nq][h1]; they become rows [pos, pos + nq) of every request.
void or_kv_append(int b, int nq, int h1, int heads, int pos, const uint16_t* k_rows,
                  const uint16_t* v_rows, int kv_fmt, int cap, void* k_store, void* v_store,
                  uint16_t* k_sm, uint16_t* v_sm) {
  const int d = h1 / heads;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < b; ++r) {
    kv_store(kv_fmt, heads, d, cap, r, pos, nq, k_rows + (i64)r * nq * h1, h1, k_store, k_sm);
    kv_store(kv_fmt, heads, d, cap, r, pos, nq, v_rows + (i64)r * nq * h1, h1, v_store, v_sm);
  }
}

// Read rows [0, T) of request r, head h, as fp16 values dst[T][d].
static void kv_load(int fmt, int H, int d, int cap, int r, int h, int T, const void* store,
                    const uint16_t* sm, uint16_t* dst) {
  for (int j = 0; j < T; ++j) {
    const i64 row = ((i64)r * H + h) * cap + j;
    if (fmt == OR_F16) {
      std::memcpy(dst + (i64)j * d, (const uint16_t*)store + row * d, sizeof(uint16_t) * d);
    } else {
      const uint8_t* cb = (const uint8_t*)store + row * (d / 2);
      for (int c = 0; c < d; ++c) {
        const int code = (c & 1) ? (cb[c / 2] >> 4) : (cb[c / 2] & 15);
        const uint16_t* s = sm + (row * (d / 64) + c / 64) * 2;
        dst[(i64)j * d + c] = dequant_one(code, s[0], s[1]);
      }
    }
  }
}

// -------------------------------------------------------------------- layers
// The MLP and output projection shared by prefill and decode ([FlexGen]
// background section): x_out = a·wO + x; x' = relu(x_out·w1)·w2 + x_out,
// with fp16 rounding of a, x_out, relu(x_out·w1) and x'.
static void layer_tail(i64 M, int h1, int h2, const uint16_t* a, const uint16_t* x,
                       const uint16_t* wo, const uint16_t* w1, const uint16_t* w2, uint16_t* y) {
  std::vector<uint16_t> xo((size_t)(M * h1)), hd((size_t)(M * h2));
  or_gemm(a, h1, wo, M, h1, h1, x, h1, 0, xo.data(), h1);
  or_gemm(xo.data(), h1, w1, M, h1, h2, nullptr, 0, 1, hd.data(), h2);
  or_gemm(hd.data(), h2, w2, M, h2, h1, xo.data(), h1, 0, y, h1);
}

// Prefill of one layer ([FlexGen] background section, prefill equations) for
// b requests of s tokens: x[b][s][h1] -> x_next[b][s][h1], and the cache rows
// [0, s) of every request.  causal = 1 masks key j > query i (reading: the
// page leaves the mask unstated; causal is the only mask under which a
// prefill of s tokens followed by one decode step equals a prefill of s + 1
// tokens); causal = 0 is the unmasked literal form.
void or_layer_prefill(int b, int s, int h1, int h2, int heads, const uint16_t* x,
                      const uint16_t* wq, const uint16_t* wk, const uint16_t* wv,
                      const uint16_t* wo, const uint16_t* w1, const uint16_t* w2, int kv_fmt,
                      int cap, void* k_store, void* v_store, uint16_t* k_sm, uint16_t* v_sm,
                      int causal, uint16_t* x_next) {
  const i64 M = (i64)b * s;
  const int d = h1 / heads;
  std::vector<uint16_t> Q((size_t)(M * h1)), K((size_t)(M * h1)), V((size_t)(M * h1)),
      A((size_t)(M * h1));
  or_gemm(x, h1, wq, M, h1, h1, nullptr, 0, 0, Q.data(), h1);
  or_gemm(x, h1, wk, M, h1, h1, nullptr, 0, 0, K.data(), h1);
  or_gemm(x, h1, wv, M, h1, h1, nullptr, 0, 0, V.data(), h1);
  for (int r = 0; r < b; ++r) {
    kv_store(kv_fmt, heads, d, cap, r, 0, s, K.data() + (i64)r * s * h1, h1, k_store, k_sm);
    kv_store(kv_fmt, heads, d, cap, r, 0, s, V.data() + (i64)r * s * h1, h1, v_store, v_sm);
  }
  // Attention reads the fresh fp16 K and V (reading: the compressed copy is
  // what is stored for later steps).
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int r = 0; r < b; ++r)
    for (int h = 0; h < heads; ++h) {
      std::vector<int> lim(s);
      for (int i = 0; i < s; ++i) lim[i] = causal ? i + 1 : s;
      const i64 off = (i64)r * s * h1 + (i64)h * d;
      attn_rows(d, s, Q.data() + off, h1, K.data() + off, V.data() + off, h1, lim.data(),
                nullptr, 0, A.data() + off, h1);
    }
  layer_tail(M, h1, h2, A.data(), x, wo, w1, w2, x_next);
}

// Decode of one layer ([FlexGen] background section, decode equations) for b
// requests, each bringing nq new tokens t[b][nq][h1] at cache rows
// [pos, pos + nq).  The new K/V rows are concatenated to the cache first; the
// queries then read every visible row through the stored format (reading:
// update, then compute, as the page orders the two steps).  masks == null:
// token i sees rows [0, pos + i] (a chain).  Otherwise masks[r][i] lists the
// new rows token i sees ([SpecPipe] 2.2.1-2.2.2: the tree mask replaces the
// causal mask), on top of all rows [0, pos).
void or_layer_decode(int b, int nq, int h1, int h2, int heads, int pos, const uint64_t* masks,
                     const uint16_t* t, const uint16_t* wq, const uint16_t* wk,
                     const uint16_t* wv, const uint16_t* wo, const uint16_t* w1,
                     const uint16_t* w2, int kv_fmt, int cap, void* k_store, void* v_store,
                     uint16_t* k_sm, uint16_t* v_sm, uint16_t* t_next) {
  const i64 M = (i64)b * nq;
  const int d = h1 / heads;
  std::vector<uint16_t> Q((size_t)(M * h1)), K((size_t)(M * h1)), V((size_t)(M * h1)),
      A((size_t)(M * h1));
  or_gemm(t, h1, wq, M, h1, h1, nullptr, 0, 0, Q.data(), h1);
  or_gemm(t, h1, wk, M, h1, h1, nullptr, 0, 0, K.data(), h1);
  or_gemm(t, h1, wv, M, h1, h1, nullptr, 0, 0, V.data(), h1);
  for (int r = 0; r < b; ++r) {
    kv_store(kv_fmt, heads, d, cap, r, pos, nq, K.data() + (i64)r * nq * h1, h1, k_store, k_sm);
    kv_store(kv_fmt, heads, d, cap, r, pos, nq, V.data() + (i64)r * nq * h1, h1, v_store, v_sm);
  }
  const int T = pos + nq;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int r = 0; r < b; ++r)
    for (int h = 0; h < heads; ++h) {
      std::vector<uint16_t> kk((size_t)T * d), vv((size_t)T * d);
      kv_load(kv_fmt, heads, d, cap, r, h, T, k_store, k_sm, kk.data());
      kv_load(kv_fmt, heads, d, cap, r, h, T, v_store, v_sm, vv.data());
      std::vector<int> lim(nq);
      for (int i = 0; i < nq; ++i) lim[i] = masks ? pos : pos + i + 1;
      const i64 off = (i64)r * nq * h1 + (i64)h * d;
      attn_rows(d, nq, Q.data() + off, h1, kk.data(), vv.data(), d, lim.data(),
                masks ? masks + (i64)r * nq : nullptr, pos, A.data() + off, h1);
    }
  layer_tail(M, h1, h2, A.data(), t, wo, w1, w2, t_next);
}

// ------------------------------------------------------------- tree masks
// [SpecPipe] 2.2.1 (layer appending, Fig. 5-a): tokens are listed in BFS
// order and each sees itself and its ancestors.  Bit u of mask[i] is set iff
// token u lies on the path from token i up to the root, found by walking the
// parent links (parent = -1 ends the walk).  Returns 0, or -1 if a parent
// does not precede its child (then masks are unspecified).
int or_tree_masks(const int32_t* parent, int nq, uint64_t* mask) {
  if (nq < 1 || nq > 64) return -1;
  for (int i = 0; i < nq; ++i)
    if (parent[i] >= i || parent[i] < -1 || (i == 0 && parent[i] != -1)) return -1;
  for (int i = 0; i < nq; ++i) {
    uint64_t m = 0;
    for (int u = i; u >= 0; u = parent[u]) m |= 1ull << u;
    mask[i] = m;
  }
  return 0;
}

// ------------------------------------------------------------ tree pruning
// [SpecPipe] 2.2.1 (sub-tree pruning, Fig. 5-b) and 2.2.2 (Fig. 8).  When
// token u is verified, column u of the mask matrix M selects the tokens whose
// path to the root passes through u: u and its descendants.  The token arrays
// keep exactly those tokens, in their BFS order, and the new mask makes u the
// root.  The cache keeps the rows of the verified path above u (the root down
// to u's parent, found as row u of M without u itself): they leave the tree
// and join the committed prefix.
// Outputs: *depth = length of that path (rows committed to the prefix);
// src[j] for j < depth + kept = old index of the token whose cache row goes
// to position j after the old prefix: the path (root first), then the kept
// tokens; src[j] = -1 beyond.  new_parent[t] for t < kept = the new index of
// kept token t's parent (-1 for u); slots t >= kept hold filler leaves (the
// parent of the last kept token, or 0 when u is the only one) so that the
// array stays a valid BFS parent array.  Returns kept, or -1 when the parent
// array is invalid or u is outside [0, nq).
int or_tree_prune(const int32_t* parent, int nq, int u, int32_t* new_parent, int32_t* src,
                  int32_t* depth) {
  uint64_t mask[64];
  if (or_tree_masks(parent, nq, mask) != 0 || u < 0 || u >= nq) return -1;
  // the verified path above u: row u of M, less u itself, in index order
  int path = 0;
  for (int i = 0; i < u; ++i)
    if ((mask[u] >> i) & 1ull) src[path++] = i;
  // the kept tokens: column u of M, in index (BFS) order, u first
  int newidx[64];
  int kept = 0;
  for (int i = 0; i < nq; ++i) {
    newidx[i] = -1;
    if ((mask[i] >> u) & 1ull) {
      newidx[i] = kept;
      src[path + kept] = i;
      ++kept;
    }
  }
  for (int t = 0; t < kept; ++t) {
    const int i = src[path + t];
    new_parent[t] = i == u ? -1 : newidx[parent[i]];
  }
  const int fill = kept == 1 ? 0 : new_parent[kept - 1];
  for (int t = kept; t < nq; ++t) new_parent[t] = fill;
  for (int j = path + kept; j < nq; ++j) src[j] = -1;
  *depth = path;
  return kept;
}

// ------------------------------------------------------------ block schedule
// [FlexGen] section 4 (computation schedule, Algorithm 1 and Fig. 3): a block
// of b = gbs x (b / gbs) requests; generation step i = 0 is the prefill
// column, steps 1..n are decode columns.  order 0 is the zig-zag block
// schedule: for step i, for layer j, for GPU batch k.  order 1 is the
// row-by-row schedule of the baseline systems: for GPU batch k, for step i,
// for layer j.  order 2 is the diagonal block schedule ([FlexGen] appendix
// A.2, Fig. 5): GPU batch k starts one iteration after batch k - 1, so at
// iteration it batch k is at step it - k (0 <= it - k <= n); each iteration
// runs layer 0 for every batch on that diagonal, then layer 1, and so on.
// Each layer's K/V cache lives in kv_k[j], kv_v[j] (and the sm arrays for
// int4); under order 2 a batch needs its cache only from its prefill to its
// last step, so batch k uses cache slot k mod min(nb, n + 1) (the arrays hold
// that many GPU batches).  Inputs: x[b][s][h1] (prompt embeddings) and
// t_in[n][b][h1] (one embedding per decode step: the pages define no token
// sampling, so each decode step is fed a given embedding).  Outputs: the last
// layer's prefill activations x_out[b][s][h1] and decode outputs
// t_out[n][b][h1].  Weights w[j * 6 + {0..5}] = wq, wk, wv, wo, w1, w2 of
// layer j, fp16 values.
void or_run_block(int b, int s, int n, int h1, int h2, int l, int heads, int gbs, int order,
                  const uint16_t* x, const uint16_t* t_in, const uint16_t* const* w, int kv_fmt,
                  int cap, void* const* kv_k, void* const* kv_v, uint16_t* const* k_sm,
                  uint16_t* const* v_sm, uint16_t* x_out, uint16_t* t_out) {
  const int nb = b / gbs;
  const int d = h1 / heads;
  const i64 code_row = kv_fmt == OR_F16 ? (i64)d * 2 : d / 2;  // bytes per cache row
  const i64 sm_row = kv_fmt == OR_F16 ? 0 : (d / 64) * 2;    // uint16 per cache row
  const i64 req_rows = (i64)heads * cap;
  // per-micro-batch activations (prefill and decode)
  std::vector<std::vector<uint16_t>> xa(nb), ta(nb);
  const int nslot = order == 2 ? std::min(nb, n + 1) : nb;
  auto run = [&](int i, int j, int k) {
    const i64 r0 = (i64)k * gbs;
    const i64 c0 = (i64)(k % nslot) * gbs;  // first request of this batch's cache slot
    void* kk = (uint8_t*)kv_k[j] + c0 * req_rows * code_row;
    void* vv = (uint8_t*)kv_v[j] + c0 * req_rows * code_row;
    uint16_t* ks = kv_fmt == OR_F16 ? nullptr : k_sm[j] + c0 * req_rows * sm_row;
    uint16_t* vs = kv_fmt == OR_F16 ? nullptr : v_sm[j] + c0 * req_rows * sm_row;
    const uint16_t* const* W = w + 6 * j;
    if (i == 0) {
      std::vector<uint16_t>& cur = xa[k];
      if (j == 0) cur.assign(x + r0 * s * h1, x + (r0 + gbs) * s * h1);
      std::vector<uint16_t> nxt(cur.size());
      or_layer_prefill(gbs, s, h1, h2, heads, cur.data(), W[0], W[1], W[2], W[3], W[4], W[5],
                       kv_fmt, cap, kk, vv, ks, vs, 1, nxt.data());
      cur.swap(nxt);
      if (j == l - 1) std::memcpy(x_out + r0 * s * h1, cur.data(), cur.size() * 2);
    } else {
      std::vector<uint16_t>& cur = ta[k];
      const uint16_t* src = t_in + ((i64)(i - 1) * b + r0) * h1;
      if (j == 0) cur.assign(src, src + (i64)gbs * h1);
      std::vector<uint16_t> nxt(cur.size());
      or_layer_decode(gbs, 1, h1, h2, heads, s + i - 1, nullptr, cur.data(), W[0], W[1], W[2],
                      W[3], W[4], W[5], kv_fmt, cap, kk, vv, ks, vs, nxt.data());
      cur.swap(nxt);
      if (j == l - 1)
        std::memcpy(t_out + ((i64)(i - 1) * b + r0) * h1, cur.data(), cur.size() * 2);
    }
  };
  if (order == 0) {
    for (int i = 0; i <= n; ++i)
      for (int j = 0; j < l; ++j)
        for (int k = 0; k < nb; ++k) run(i, j, k);
  } else if (order == 2) {
    for (int it = 0; it < nb + n; ++it)
      for (int j = 0; j < l; ++j)
        for (int k = std::max(0, it - n); k <= std::min(it, nb - 1); ++k) run(it - k, j, k);
  } else {
    for (int k = 0; k < nb; ++k)
      for (int i = 0; i <= n; ++i)
        for (int j = 0; j < l; ++j) run(i, j, k);
  }
}

}  // extern "C"
