// The C ABI of libhp: argument checks, the layer composition ([FlexGen]
// paper notes, background section: prefill and decode equations) and the
// zig-zag block runner ([FlexGen] section 4, Algorithm 1), with the decode
// column captured once as a hipGraph and replayed n times.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "common.h"

namespace hp {

static thread_local char g_err[512] = "";

hp_status fail(hp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

hp_status hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return HP_OK;
  return fail(HP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

hp_status launch_ok(const char* kernel) { return hip_ok(hipGetLastError(), kernel); }

// --------------------------------------------------------- small kernels
// Moves one step's rows between a [steps][...] tensor and a flat buffer:
// direction 0: dst[i] = src[step * stride + i]; direction 1: dst[step * stride
// + i] = src[i], for i < count (all in 16-byte units, step = *dstep).
__global__ __launch_bounds__(256) void k_copy_step(const uint4* __restrict__ src, int64_t count,
                                                   int64_t stride,
                                                   const int32_t* __restrict__ dstep,
                                                   uint4* __restrict__ dst, int direction) {
  const int64_t off = (int64_t)(*dstep) * stride;
  const int64_t gs = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gs) {
    if (direction == 0)
      dst[i] = src[off + i];
    else
      dst[off + i] = src[i];
  }
}

__global__ void k_set_i32(int32_t* p, int32_t v, int add) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = add ? *p + v : v;
}

void launch_copy_step(const void* src, int64_t count_elems, int64_t stride_elems,
                      const int32_t* dstep, void* dst, int direction, hipStream_t st) {
  const int64_t n16 = count_elems / 8;
  const int blocks = (int)std::min<int64_t>(cdiv(n16, 256), 4096);
  Prof prof("copy_step", st);
  hipLaunchKernelGGL(k_copy_step, dim3(blocks), dim3(256), 0, st, (const uint4*)src, n16,
                     stride_elems / 8, dstep, (uint4*)dst, direction);
}

static void launch_set_i32(int32_t* p, int32_t v, bool add, hipStream_t st) {
  hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(64), 0, st, p, v, add ? 1 : 0);
}

void launch_add_i32(int32_t* p, int32_t v, hipStream_t st) { launch_set_i32(p, v, true, st); }

// Diagonal schedule ([FlexGen] appendix A.2): the live requests r0 .. r0 + M
// of iteration it, request r in GPU batch r / gbs at decode step
// t = it - r / gbs.  direction 0: dst row i = t_in[t - 1][r] and rpos[i] =
// s + t - 1 (the row of its new token); direction 1: t_out[t - 1][r] = src
// row i.  Rows of h1 halves, 16-byte units.
__global__ __launch_bounds__(256) void k_diag_rows(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst,
                                                   int32_t* __restrict__ rpos, int M, int r0,
                                                   int gbs, int b, int s, int it, int h1,
                                                   int direction) {
  const int w = h1 / 8;  // 16-byte units per row
  const int64_t total = (int64_t)M * w;
  const int64_t gs = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gs) {
    const int i = (int)(e / w), c = (int)(e % w);
    const int r = r0 + i, t = it - r / gbs;
    const int64_t step_row = ((int64_t)(t - 1) * b + r) * w + c;
    if (direction == 0) {
      dst[(int64_t)i * w + c] = src[step_row];
      if (c == 0) rpos[i] = s + t - 1;
    } else {
      dst[step_row] = src[(int64_t)i * w + c];
    }
  }
}

static void launch_diag_rows(const void* src, void* dst, int32_t* rpos, int M, int r0, int gbs,
                             int b, int s, int it, int h1, int direction, hipStream_t st) {
  const int64_t units = (int64_t)M * (h1 / 8);
  const int blocks = (int)std::min<int64_t>(cdiv(units, 256), 4096);
  Prof prof("diag_rows", st);
  hipLaunchKernelGGL(k_diag_rows, dim3(blocks), dim3(256), 0, st, (const uint4*)src, (uint4*)dst,
                     rpos, M, r0, gbs, b, s, it, h1, direction);
}

// [FlexGen] appendix A.2 (diagonal block schedule): the cache pages of
// page_rows rows that each request holds, when every live request keeps
// only the pages its current length needs.  Request r of GPU batch k takes
// the pages of rows [0, s) at its prefill (iteration k) and, at decode step t
// (iteration k + t), those of rows up to s + t; after its last step (t = n)
// its batch's pages return to the pool.  Free pages go out lowest index
// first.  Fills table [b][cap / page_rows] (-1: never used) if given and
// returns the peak count of pages in use.
static int64_t diag_page_plan(const hp_dims& d, int page_rows, int cap,
                              std::vector<int32_t>* table) {
  const int nb = d.b / d.gbs, ppr = cap / page_rows;
  std::vector<int32_t> tb((size_t)d.b * ppr, -1);
  std::vector<int> held((size_t)d.b, 0);
  std::set<int32_t> free_pages;
  int32_t next = 0;
  int64_t used = 0, peak = 0;
  auto grow = [&](int k, int rows) {
    const int need = (int)cdiv(rows, page_rows);
    for (int i = 0; i < d.gbs; ++i) {
      const int64_t r = (int64_t)k * d.gbs + i;
      for (; held[r] < need; ++held[r], ++used) {
        int32_t p = next;
        if (!free_pages.empty()) {
          p = *free_pages.begin();
          free_pages.erase(free_pages.begin());
        } else {
          ++next;
        }
        tb[(size_t)r * ppr + held[r]] = p;
      }
    }
  };
  for (int it = 0; it < nb + d.n; ++it) {
    if (it < nb) grow(it, d.s);
    for (int k = std::max(0, it - d.n); k <= std::min(it - 1, nb - 1); ++k) grow(k, d.s + (it - k));
    peak = std::max(peak, used);
    const int k = it - d.n;  // batch whose last decode step was this iteration
    if (k >= 0 && k < nb) {
      for (int i = 0; i < d.gbs; ++i) {
        const int64_t r = (int64_t)k * d.gbs + i;
        for (int pg = 0; pg < held[r]; ++pg) free_pages.insert(tb[(size_t)r * ppr + pg]);
        used -= held[r];
      }
    }
  }
  if (table) table->swap(tb);
  return peak;
}

// ---------------------------------------------------------------- checks
static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
#define NEED_ALIGN(p, a)                                                              \
  do {                                                                                \
    if (!aligned((p), (a))) return fail(HP_ERR_SHAPE, "%s must be %d-byte aligned", #p, (int)(a)); \
  } while (0)

static int g_dev_ok[64];  // 0 unknown, 1 gfx950, -1 other

static hp_status device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(HP_ERR_DEVICE, "no HIP device");
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(HP_ERR_DEVICE, "no HIP device");
    g_dev_ok[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (g_dev_ok[dev] != 1) return fail(HP_ERR_DEVICE, "device is not gfx950");
  return HP_OK;
}

static hp_status check_dims(const hp_dims* d) {
  if (!d) return fail(HP_ERR_NULL, "dims is NULL");
  if (d->b <= 0 || d->s <= 0 || d->n < 0 || d->h1 <= 0 || d->h2 <= 0 || d->l <= 0 ||
      d->heads <= 0 || d->gbs <= 0)
    return fail(HP_ERR_SHAPE, "dims must be positive (b=%d s=%d n=%d h1=%d h2=%d l=%d heads=%d gbs=%d)",
                d->b, d->s, d->n, d->h1, d->h2, d->l, d->heads, d->gbs);
  if (d->h1 % d->heads) return fail(HP_ERR_SHAPE, "h1 %% heads != 0");
  const int D = d->h1 / d->heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (d->h1 % 128 || d->h2 % 128) return fail(HP_ERR_SHAPE, "h1 and h2 must be multiples of 128");
  if (d->b % d->gbs) return fail(HP_ERR_SHAPE, "b %% gbs != 0");
  return HP_OK;
}

static hp_status check_mat(const hp_mat& m, int k, int n, const char* name) {
  if (m.fmt != HP_F16 && m.fmt != HP_Q4) return fail(HP_ERR_SHAPE, "%s: bad format %d", name, m.fmt);
  if (m.k != k || m.n != n)
    return fail(HP_ERR_SHAPE, "%s: shape %dx%d, expected %dx%d", name, m.k, m.n, k, n);
  if (m.k % 128 || m.n % 64) return fail(HP_ERR_SHAPE, "%s: k %% 128 or n %% 64 != 0", name);
  if (!m.data) return fail(HP_ERR_NULL, "%s: data is NULL", name);
  if (m.fmt == HP_Q4 && (!m.scale || !m.minv)) return fail(HP_ERR_NULL, "%s: scale/minv NULL", name);
  if (!aligned(m.data, 16) || (m.fmt == HP_Q4 && (!aligned(m.scale, 16) || !aligned(m.minv, 16))))
    return fail(HP_ERR_SHAPE, "%s: buffers must be 16-byte aligned", name);
  return HP_OK;
}

static hp_status check_layer(const hp_layer& w, int h1, int h2) {
  hp_status s;
  if ((s = check_mat(w.wqkv, h1, 3 * h1, "wqkv")) != HP_OK) return s;
  if ((s = check_mat(w.wo, h1, h1, "wo")) != HP_OK) return s;
  if ((s = check_mat(w.w1, h1, h2, "w1")) != HP_OK) return s;
  if ((s = check_mat(w.w2, h2, h1, "w2")) != HP_OK) return s;
  return HP_OK;
}

// Decode attention with q new tokens runs on the streaming kernel (which
// reads paged caches) unless the cache is int4 and q >= 16 (multi-query MFMA
// kernel).
static bool streaming_attention(const hp_kv* kv, int q) { return kv->fmt != HP_Q4 || q < 16; }

// paged: 0 = contiguous caches only; 1 = paged caches with a page table
// also accepted; 2 = a page pool whose table the library fills (pages NULL).
static hp_status check_kv(const hp_kv* kv, int need_rows, int paged = 0) {
  if (!kv) return fail(HP_ERR_NULL, "kv is NULL");
  if (kv->fmt != HP_F16 && kv->fmt != HP_Q4) return fail(HP_ERR_SHAPE, "kv: bad format");
  if (!kv->k || !kv->v) return fail(HP_ERR_NULL, "kv: k/v NULL");
  if (kv->fmt == HP_Q4 && (!kv->k_sm || !kv->v_sm)) return fail(HP_ERR_NULL, "kv: sm NULL");
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16) ||
      (kv->fmt == HP_Q4 && (!aligned(kv->k_sm, 4) || !aligned(kv->v_sm, 4))))
    return fail(HP_ERR_SHAPE, "kv: buffers must be 16-byte aligned (sm 4-byte)");
  if (kv->cap <= 0 || need_rows > kv->cap)
    return fail(HP_ERR_CAPACITY, "kv: %d rows needed, cap %d", need_rows, kv->cap);
  if (kv->page_rows == 0) {
    if (kv->pages || kv->pool_pages) return fail(HP_ERR_SHAPE, "kv: pages set with page_rows 0");
    return HP_OK;
  }
  if (paged == 0) return fail(HP_ERR_SHAPE, "kv: this call takes contiguous caches only");
  if (kv->page_rows < 64 || (kv->page_rows & (kv->page_rows - 1)) || kv->cap % kv->page_rows ||
      kv->pool_pages <= 0)
    return fail(HP_ERR_SHAPE, "kv: page_rows must be a power of two >= 64 dividing cap, "
                "pool_pages positive (page_rows %d, cap %d, pool %d)", kv->page_rows, kv->cap,
                kv->pool_pages);
  if (paged == 1 && !kv->pages) return fail(HP_ERR_NULL, "kv: paged cache without a page table");
  if (paged == 2 && kv->pages) return fail(HP_ERR_SHAPE, "kv: the page table of a pool is the library's");
  if (paged == 1) NEED_ALIGN(kv->pages, 4);
  return HP_OK;
}

// ---------------------------------------------------------------- workspace
struct Ws {
  size_t qkv, a, xo, hid, part, xb, t0, t1, ctr, pt, rpos, total;
};

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

static Ws ws_layout(const hp_dims& d) {
  const size_t Mp = (size_t)d.b * d.s, Md = (size_t)d.b * 64;
  const size_t M = std::max(Mp, Md);
  const int64_t Msk = std::min<int64_t>((int64_t)M, 144);
  // split-k partials of skinny products, or the fp16 expansion of an int4
  // weight for tall ones (whichever is larger)
  size_t part = 0;
  for (int64_t mm : {Msk, (int64_t)145}) {
    part = std::max(part, gemm_ws_bytes(mm, d.h1, 3 * d.h1, HP_Q4));
    part = std::max(part, gemm_ws_bytes(mm, d.h1, d.h1, HP_Q4));
    part = std::max(part, gemm_ws_bytes(mm, d.h1, d.h2, HP_Q4));
    part = std::max(part, gemm_ws_bytes(mm, d.h2, d.h1, HP_Q4));
  }
  Ws w;
  size_t o = 0;
  w.qkv = o; o += al(M * 3 * d.h1 * 2);
  w.a = o;   o += al(M * d.h1 * 2);
  w.xo = o;  o += al(M * d.h1 * 2);
  w.hid = o; o += al(M * pad_ld(d.h2) * 2);
  w.part = o; o += al(part);
  w.xb = o;  o += al(Mp * d.h1 * 2);
  w.t0 = o;  o += al(Md * d.h1 * 2);
  w.t1 = o;  o += al(Md * d.h1 * 2);
  w.ctr = o; o += 256;
  // diagonal schedule with paged caches: page table [b][ceil((s + n) / 64)]
  // (pages of at least 64 rows) and one row position per request
  w.pt = o;  o += al((size_t)d.b * cdiv(d.s + d.n, 64) * 4);
  w.rpos = o; o += al((size_t)d.b * 4);
  w.total = o;
  return w;
}

template <class T>
static T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// ---------------------------------------------------------- layer bodies
// No argument checks here: callers validated everything.
static hp_status layer_tail(const hp_layer& w, int64_t M, int h1, int h2, const void* resid,
                            void* out, void* ws, const Ws& L, hipStream_t st) {
  hp_status s;
  _Float16* a = at<_Float16>(ws, L.a);
  _Float16* xo = at<_Float16>(ws, L.xo);
  _Float16* hid = at<_Float16>(ws, L.hid);
  void* part = at<void>(ws, L.part);
  if ((s = launch_gemm(a, h1, w.wo, M, resid, h1, false, xo, h1, part, st)) != HP_OK) return s;
  const int64_t ldh = pad_ld(h2);
  if ((s = launch_gemm(xo, h1, w.w1, M, nullptr, 0, true, hid, ldh, part, st)) != HP_OK) return s;
  return launch_gemm(hid, ldh, w.w2, M, xo, h1, false, out, h1, part, st);
}

static hp_status prefill_body(int b, int s, int h1, int h2, int heads, const hp_layer& w,
                              const void* x, const hp_kv& kv, void* x_out, void* ws, const Ws& L,
                              hipStream_t st) {
  const int64_t M = (int64_t)b * s;
  _Float16* qkv = at<_Float16>(ws, L.qkv);
  hp_status r;
  if ((r = launch_gemm(x, h1, w.wqkv, M, nullptr, 0, false, qkv, 3 * h1, at<void>(ws, L.part), st)) !=
      HP_OK)
    return r;
  launch_kv_append(b, s, h1, heads, qkv, 0, nullptr, nullptr, kv, st);
  if ((r = launch_ok("k_kv_append")) != HP_OK) return r;
  launch_prefill_attention(b, s, h1, heads, qkv, at<void>(ws, L.a), st);
  if ((r = launch_ok("k_prefill_attn")) != HP_OK) return r;
  return layer_tail(w, M, h1, h2, x, x_out, ws, L, st);
}

// topk_max_t > 0: Top-K sparse attention ([FlexGen] section 5) keeping
// ceil(T / 10) rows, with T <= topk_max_t (q == 1 only).
// rpos (device int32 [b], may be NULL): each request's own row for its new
// token (at most pos); the attention then sees that request's rows up to it.
static hp_status decode_body(int b, int q, int h1, int h2, int heads, const hp_layer& w,
                             const void* t, int pos, const int32_t* dpos, const uint64_t* masks,
                             const hp_kv& kv, void* t_out, void* ws, const Ws& L, hipStream_t st,
                             int topk_max_t = 0, const int32_t* rpos = nullptr) {
  const int64_t M = (int64_t)b * q;
  _Float16* qkv = at<_Float16>(ws, L.qkv);
  hp_status r;
  if ((r = launch_gemm(t, h1, w.wqkv, M, nullptr, 0, false, qkv, 3 * h1, at<void>(ws, L.part), st)) !=
      HP_OK)
    return r;
  launch_kv_append(b, q, h1, heads, qkv, pos, dpos, rpos, kv, st);
  if ((r = launch_ok("k_kv_append")) != HP_OK) return r;
  if (topk_max_t > 0) {
    if ((r = launch_topk_attention(b, h1, heads, qkv, pos, dpos, topk_max_t, 0, kv,
                                   at<void>(ws, L.a), nullptr, st, rpos)) != HP_OK)
      return fail(r, "topk attention: bad row count");
    if ((r = launch_ok("k_topk_attn")) != HP_OK) return r;
  } else {
    launch_decode_attention(b, q, h1, heads, qkv, pos, dpos, rpos, masks, kv, at<void>(ws, L.a),
                            st);
    if ((r = launch_ok("k_decode_attn")) != HP_OK) return r;
  }
  return layer_tail(w, M, h1, h2, t, t_out, ws, L, st);
}

// Cache view of requests [r0, r0 + nb) of a layer's cache.
static hp_kv kv_slice(const hp_kv& kv, int heads, int D, int64_t r0) {
  hp_kv o = kv;
  if (kv.page_rows > 0) {  // the same pool; these requests' rows of the page table
    o.pages = kv.pages + r0 * (kv.cap / kv.page_rows);
    return o;
  }
  const int64_t rows = r0 * heads * kv.cap;
  if (kv.fmt == HP_F16) {
    o.k = (char*)kv.k + rows * D * 2;
    o.v = (char*)kv.v + rows * D * 2;
  } else {
    o.k = (char*)kv.k + rows * (D / 2);
    o.v = (char*)kv.v + rows * (D / 2);
    o.k_sm = (char*)kv.k_sm + rows * (D / 64) * 4;
    o.v_sm = (char*)kv.v_sm + rows * (D / 64) * 4;
  }
  return o;
}

// Layer of the decode cells of one diagonal ([FlexGen] appendix A.2): GPU
// batches c = 0..nbat-1 of gbs requests each, rows contiguous in t / t_out,
// batch c at cache row pos[c] of cache slot slot[c].  One QKV product and one
// tail for all of them (each weight matrix read once), append and attention
// per batch.
static hp_status decode_cells(int gbs, int nbat, const int* pos, const int* slot, int h1, int h2,
                              int heads, const hp_layer& w, const void* t, const hp_kv& kv,
                              void* t_out, void* ws, const Ws& L, hipStream_t st,
                              int topk_max_t) {
  const int64_t M = (int64_t)gbs * nbat;
  const int D = h1 / heads;
  _Float16* qkv = at<_Float16>(ws, L.qkv);
  _Float16* att = at<_Float16>(ws, L.a);
  hp_status r;
  if ((r = launch_gemm(t, h1, w.wqkv, M, nullptr, 0, false, qkv, 3 * h1, at<void>(ws, L.part), st)) !=
      HP_OK)
    return r;
  for (int c = 0; c < nbat; ++c) {
    const _Float16* qc = qkv + (int64_t)c * gbs * 3 * h1;
    const hp_kv kc = kv_slice(kv, heads, D, (int64_t)slot[c] * gbs);
    launch_kv_append(gbs, 1, h1, heads, qc, pos[c], nullptr, nullptr, kc, st);
    if ((r = launch_ok("k_kv_append")) != HP_OK) return r;
    _Float16* ac = att + (int64_t)c * gbs * h1;
    if (topk_max_t > 0) {
      if ((r = launch_topk_attention(gbs, h1, heads, qc, pos[c], nullptr, topk_max_t, 0, kc, ac,
                                     nullptr, st)) != HP_OK)
        return fail(r, "topk attention: bad row count");
      if ((r = launch_ok("k_topk_attn")) != HP_OK) return r;
    } else {
      launch_decode_attention(gbs, 1, h1, heads, qc, pos[c], nullptr, nullptr, nullptr, kc, ac, st);
      if ((r = launch_ok("k_decode_attn")) != HP_OK) return r;
    }
  }
  return layer_tail(w, M, h1, h2, t, t_out, ws, L, st);
}

// -------------------------------------------------------------- profiling
static std::mutex g_pmu;
static bool g_prof = false;
static std::vector<std::pair<std::string, std::pair<hipEvent_t, hipEvent_t>>> g_prec;
static std::vector<hipEvent_t> g_pool;

static hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

Prof::Prof(const char* t, hipStream_t s) : tag(t), st(s) {
  if (!g_prof) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  std::lock_guard<std::mutex> lk(g_pmu);
  a = pool_event();
  b = pool_event();
  // best effort: a failed record only loses this sample
  if (a && b) (void)hipEventRecord(a, st);
}

Prof::~Prof() {
  if (!a || !b) return;
  (void)hipEventRecord(b, st);
  std::lock_guard<std::mutex> lk(g_pmu);
  g_prec.push_back({tag, {a, b}});
}

// ----------------------------------------------------------------- graphs
static std::mutex g_mu;
static std::map<std::vector<uint64_t>, hipGraphExec_t> g_graphs;

}  // namespace hp

using namespace hp;

extern "C" {

const char* hp_last_error(void) { return g_err; }

hp_status hp_device_check(void) { return device_check(); }

hp_status hp_quantize_g64(const void* x, int64_t rows, int64_t cols, void* codes, void* sm,
                          void* stream) {
  if (rows < 0 || cols <= 0 || cols % 64) return fail(HP_ERR_SHAPE, "cols must be a positive multiple of 64, rows >= 0");
  if (rows == 0) return HP_OK;
  if (!x || !codes || !sm) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(x, 16);
  NEED_ALIGN(codes, 4);
  NEED_ALIGN(sm, 4);
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_quantize_g64(x, rows, cols, codes, sm, S(stream));
  return launch_ok("k_quantize_g64");
}

hp_status hp_dequantize_g64(const void* codes, const void* sm, int64_t rows, int64_t cols, void* y,
                            void* stream) {
  if (rows < 0 || cols <= 0 || cols % 64) return fail(HP_ERR_SHAPE, "cols must be a positive multiple of 64, rows >= 0");
  if (rows == 0) return HP_OK;
  if (!y || !codes || !sm) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(y, 16);
  NEED_ALIGN(codes, 4);
  NEED_ALIGN(sm, 4);
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_dequantize_g64(codes, sm, rows, cols, y, S(stream));
  return launch_ok("k_dequantize_g64");
}

hp_status hp_pack_weight_q4(const void* codes, const void* sm, int32_t k, int32_t n, void* packed,
                            void* scale, void* minv, void* stream) {
  if (k <= 0 || n <= 0 || k % 128 || n % 64) return fail(HP_ERR_SHAPE, "need k %% 128 == 0, n %% 64 == 0");
  if (!codes || !sm || !packed || !scale || !minv) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(sm, 4);
  NEED_ALIGN(packed, 4);
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_pack_q4(codes, sm, k, n, packed, scale, minv, S(stream));
  return launch_ok("k_pack_q4");
}

hp_status hp_pack_weight_f16(const void* w, int32_t k, int32_t n, void* wt, void* stream) {
  if (k <= 0 || n <= 0 || k % 128 || n % 64) return fail(HP_ERR_SHAPE, "need k %% 128 == 0, n %% 64 == 0");
  if (!w || !wt) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(wt, 16);
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_pack_f16(w, k, n, wt, S(stream));
  return launch_ok("k_pack_f16");
}

size_t hp_gemm_workspace_bytes(int64_t M, int32_t k, int32_t n, int32_t fmt) {
  if (M <= 0 || k <= 0 || n <= 0 || k % 128) return 0;
  return gemm_ws_bytes(M, k, n, fmt);
}

hp_status hp_gemm(const void* x, int64_t ldx, const hp_mat* w, int64_t M, const void* res,
                  int64_t ldr, int32_t relu, void* y, int64_t ldy, void* ws, size_t ws_bytes,
                  void* stream) {
  if (!w) return fail(HP_ERR_NULL, "w is NULL");
  if (M < 0) return fail(HP_ERR_SHAPE, "M < 0");
  hp_status s = check_mat(*w, w->k, w->n, "w");
  if (s != HP_OK) return s;
  if (M == 0) return HP_OK;
  if (!x || !y) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(x, 16);
  NEED_ALIGN(y, 8);
  if (res) NEED_ALIGN(res, 8);
  if (ws) NEED_ALIGN(ws, 16);
  if (ldx < w->k || ldx % 8 || ldy < w->n || ldy % 4 || (res && (ldr < w->n || ldr % 4)))
    return fail(HP_ERR_SHAPE, "row strides too small or misaligned");
  const size_t need = gemm_ws_bytes(M, w->k, w->n, w->fmt);
  if (ws_bytes < need || (need && !ws))
    return fail(HP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((s = device_check()) != HP_OK) return s;
  return launch_gemm(x, ldx, *w, M, res, ldr, relu != 0, y, ldy, ws, S(stream));
}

hp_status hp_gemm_noalloc(const void* x, int64_t ldx, const hp_mat* w, int64_t M,
                          const void* res, int64_t ldr, int32_t relu, void* y, int64_t ldy,
                          void* stream) {
  if (!w) return fail(HP_ERR_NULL, "w is NULL");
  if (M < 0) return fail(HP_ERR_SHAPE, "M < 0");
  hp_status s = check_mat(*w, w->k, w->n, "w");
  if (s != HP_OK) return s;
  if (M == 0) return HP_OK;
  if (M > kSkinnyM)
    return fail(HP_ERR_SHAPE, "hp_gemm_noalloc takes M <= %d rows (M = %lld); taller products "
                "need a weight-sized buffer: use hp_gemm", (int)kSkinnyM, (long long)M);
  if (!x || !y) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(x, 16);
  NEED_ALIGN(y, 8);
  if (res) NEED_ALIGN(res, 8);
  if (ldx < w->k || ldx % 8 || ldy < w->n || ldy % 4 || (res && (ldr < w->n || ldr % 4)))
    return fail(HP_ERR_SHAPE, "row strides too small or misaligned");
  const size_t need = gemm_ws_bytes(M, w->k, w->n, w->fmt);
  if (need > kStaticScratchBytes)
    return fail(HP_ERR_WORKSPACE, "product needs %zu bytes of split partials, above the %zu-byte "
                "static scratch", need, kStaticScratchBytes);
  if ((s = device_check()) != HP_OK) return s;
  void* ws = nullptr;
  if ((s = static_scratch(&ws)) != HP_OK) return s;
  return launch_gemm(x, ldx, *w, M, res, ldr, relu != 0, y, ldy, ws, S(stream));
}

hp_status hp_kv_append(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                       int32_t pos, const hp_kv* kv, void* stream) {
  if (b <= 0 || q <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || pos < 0)
    return fail(HP_ERR_SHAPE, "bad sizes");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!qkv) return fail(HP_ERR_NULL, "qkv is NULL");
  NEED_ALIGN(qkv, 16);
  hp_status s = check_kv(kv, pos + q, 1);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  launch_kv_append(b, q, h1, heads, qkv, pos, nullptr, nullptr, *kv, S(stream));
  return launch_ok("k_kv_append");
}

hp_status hp_kv_append_ragged(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                              const int32_t* rpos, int32_t max_pos, const hp_kv* kv,
                              void* stream) {
  if (b <= 0 || q <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || max_pos < 0)
    return fail(HP_ERR_SHAPE, "bad sizes");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!qkv || !rpos) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(qkv, 16);
  NEED_ALIGN(rpos, 4);
  hp_status s = check_kv(kv, max_pos + q, 1);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  launch_kv_append(b, q, h1, heads, qkv, max_pos, nullptr, rpos, *kv, S(stream));
  return launch_ok("k_kv_append");
}

hp_status hp_prefill_attention(int32_t b, int32_t s_, int32_t h1, int32_t heads, const void* qkv,
                               void* out, void* stream) {
  if (b <= 0 || s_ <= 0 || h1 <= 0 || heads <= 0 || h1 % heads) return fail(HP_ERR_SHAPE, "bad sizes");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!qkv || !out) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(qkv, 16);
  NEED_ALIGN(out, 16);
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_prefill_attention(b, s_, h1, heads, qkv, out, S(stream));
  return launch_ok("k_prefill_attn");
}

hp_status hp_decode_attention(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                              int32_t pos, const uint64_t* masks, const hp_kv* kv, void* out,
                              void* stream) {
  if (b <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || pos < 0) return fail(HP_ERR_SHAPE, "bad sizes");
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!qkv || !out) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(qkv, 16);
  NEED_ALIGN(out, 16);
  if (masks) NEED_ALIGN(masks, 8);
  hp_status s = check_kv(kv, pos + q, kv && streaming_attention(kv, q) ? 1 : 0);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  launch_decode_attention(b, q, h1, heads, qkv, pos, nullptr, nullptr, masks, *kv, out, S(stream));
  return launch_ok("k_decode_attn");
}

hp_status hp_decode_attention_ragged(int32_t b, int32_t q, int32_t h1, int32_t heads,
                                     const void* qkv, const int32_t* prefix, int32_t max_prefix,
                                     const uint64_t* masks, const hp_kv* kv, void* out,
                                     void* stream) {
  if (b <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || max_prefix < 0)
    return fail(HP_ERR_SHAPE, "bad sizes");
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!qkv || !out || !prefix) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(qkv, 16);
  NEED_ALIGN(out, 16);
  NEED_ALIGN(prefix, 4);
  if (masks) NEED_ALIGN(masks, 8);
  hp_status s = check_kv(kv, max_prefix + q, kv && streaming_attention(kv, q) ? 1 : 0);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  launch_decode_attention(b, q, h1, heads, qkv, max_prefix, nullptr, prefix, masks, *kv, out,
                          S(stream));
  return launch_ok("k_decode_attn");
}

hp_status hp_topk_attention(int32_t b, int32_t h1, int32_t heads, const void* qkv, int32_t pos,
                            int32_t topk, const hp_kv* kv, void* out, int32_t* idx, void* stream) {
  if (b <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || pos < 0) return fail(HP_ERR_SHAPE, "bad sizes");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (pos + 1 > 4096) return fail(HP_ERR_SHAPE, "pos + 1 = %d rows exceeds 4096", pos + 1);
  if (topk < 0) return fail(HP_ERR_SHAPE, "topk must be >= 0");
  if (!qkv || !out) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(qkv, 16);
  NEED_ALIGN(out, 16);
  hp_status s = check_kv(kv, pos + 1, 1);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  if ((s = launch_topk_attention(b, h1, heads, qkv, pos, nullptr, pos + 1, topk, *kv, out, idx,
                                 S(stream))) != HP_OK)
    return fail(s, "topk attention: bad row count");
  return launch_ok("k_topk_attn");
}

hp_status hp_tree_masks(int32_t b, int32_t q, const int32_t* parent, uint64_t* masks, int32_t* err,
                        void* stream) {
  if (b <= 0) return fail(HP_ERR_SHAPE, "b must be positive");
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  if (!parent || !masks) return fail(HP_ERR_NULL, "NULL pointer");
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_tree_masks(b, q, parent, masks, err, S(stream));
  return launch_ok("k_tree_masks");
}

hp_status hp_tree_prune(int32_t b, int32_t q, const int32_t* parent, const int32_t* verified,
                        int32_t pos, int32_t* new_parent, int32_t* src, int32_t* prefix,
                        int32_t* kept, int32_t* err, void* stream) {
  if (b <= 0 || pos < 0) return fail(HP_ERR_SHAPE, "b must be positive, pos >= 0");
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  if (!parent || !verified || !new_parent || !src || !prefix || !kept)
    return fail(HP_ERR_NULL, "NULL pointer");
  hp_status s = device_check();
  if (s != HP_OK) return s;
  launch_tree_prune(b, q, pos, parent, verified, new_parent, src, prefix, kept, err, S(stream));
  return launch_ok("k_tree_prune");
}

hp_status hp_kv_compact(int32_t b, int32_t q, int32_t h1, int32_t heads, int32_t pos,
                        const int32_t* src, const int32_t* prefix, const int32_t* kept,
                        const hp_kv* kv, void* stream) {
  if (b <= 0 || h1 <= 0 || heads <= 0 || h1 % heads || pos < 0)
    return fail(HP_ERR_SHAPE, "bad sizes");
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  const int D = h1 / heads;
  if (D != 64 && D != 128) return fail(HP_ERR_SHAPE, "head dim %d not in {64, 128}", D);
  if (!src || !prefix || !kept) return fail(HP_ERR_NULL, "NULL pointer");
  hp_status s = check_kv(kv, pos + q);
  if (s != HP_OK) return s;
  if ((s = device_check()) != HP_OK) return s;
  launch_kv_compact(b, q, heads, D, pos, src, prefix, kept, *kv, S(stream));
  return launch_ok("k_kv_compact");
}

static thread_local hp_capture g_capture;
static thread_local bool g_capture_on = false;

hp_status hp_debug_set_capture(const hp_capture* c) {
  g_capture_on = c != nullptr;
  if (c) g_capture = *c;
  return HP_OK;
}

// Copies a finished layer's stored intermediates out (hp_debug_set_capture).
static hp_status capture_out(int64_t M, int h1, int h2, void* ws, const Ws& L, hipStream_t st) {
  if (!g_capture_on) return HP_OK;
  const hp_capture& c = g_capture;
  const size_t row1 = (size_t)h1 * 2;
  struct Part { void* dst; size_t src, bytes, pitch; } parts[4] = {
      {c.qkv, L.qkv, 3 * row1, 3 * row1},
      {c.attn, L.a, row1, row1},
      {c.x_out, L.xo, row1, row1},
      {c.hidden, L.hid, (size_t)h2 * 2, (size_t)pad_ld(h2) * 2}};
  for (const Part& p : parts) {
    if (!p.dst) continue;
    hp_status s = hip_ok(hipMemcpy2DAsync(p.dst, p.bytes, (const char*)ws + p.src, p.pitch, p.bytes,
                                          (size_t)M, hipMemcpyDeviceToDevice, st),
                         "capture copy");
    if (s != HP_OK) return s;
  }
  return HP_OK;
}

size_t hp_workspace_bytes(const hp_dims* d) {
  if (check_dims(d) != HP_OK) return 0;
  return ws_layout(*d).total;
}

hp_status hp_layer_prefill(const hp_dims* d, const hp_layer* w, const void* x, const hp_kv* kv,
                           void* x_out, void* ws, size_t ws_bytes, void* stream) {
  hp_status s;
  if ((s = check_dims(d)) != HP_OK) return s;
  if (!w || !x || !x_out || !ws) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(x, 16);
  NEED_ALIGN(x_out, 16);
  NEED_ALIGN(ws, 256);
  if ((s = check_layer(*w, d->h1, d->h2)) != HP_OK) return s;
  if ((s = check_kv(kv, d->s, 1)) != HP_OK) return s;
  const Ws L = ws_layout(*d);
  if (ws_bytes < L.total) return fail(HP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if ((s = device_check()) != HP_OK) return s;
  if ((s = prefill_body(d->b, d->s, d->h1, d->h2, d->heads, *w, x, *kv, x_out, ws, L,
                        S(stream))) != HP_OK)
    return s;
  return capture_out((int64_t)d->b * d->s, d->h1, d->h2, ws, L, S(stream));
}

hp_status hp_layer_decode(const hp_dims* d, const hp_layer* w, const void* t, int32_t pos,
                          int32_t q, const uint64_t* masks, const hp_kv* kv, void* t_out, void* ws,
                          size_t ws_bytes, void* stream) {
  hp_status s;
  if ((s = check_dims(d)) != HP_OK) return s;
  if (!w || !t || !t_out || !ws) return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(t, 16);
  NEED_ALIGN(t_out, 16);
  NEED_ALIGN(ws, 256);
  if (masks) NEED_ALIGN(masks, 8);
  if (q < 1 || q > 64) return fail(HP_ERR_TREE, "q must be in [1, 64]");
  if (pos < 0) return fail(HP_ERR_SHAPE, "pos < 0");
  if ((s = check_layer(*w, d->h1, d->h2)) != HP_OK) return s;
  if ((s = check_kv(kv, pos + q, kv && streaming_attention(kv, q) ? 1 : 0)) != HP_OK) return s;
  const Ws L = ws_layout(*d);
  if (ws_bytes < L.total) return fail(HP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if ((s = device_check()) != HP_OK) return s;
  if ((s = decode_body(d->b, q, d->h1, d->h2, d->heads, *w, t, pos, nullptr, masks, *kv, t_out, ws,
                       L, S(stream))) != HP_OK)
    return s;
  return capture_out((int64_t)d->b * q, d->h1, d->h2, ws, L, S(stream));
}

static void graph_key(std::vector<uint64_t>& key, const hp_dims* d, const hp_layer* layers,
                      const hp_kv* kv, const void* t_in, void* t_out, void* ws, uint32_t flags,
                      void* stream) {
  key = {(uint64_t)d->b,  (uint64_t)d->s,  (uint64_t)d->n,     (uint64_t)d->h1,
         (uint64_t)d->h2, (uint64_t)d->l,  (uint64_t)d->heads, (uint64_t)d->gbs,
         flags,           (uint64_t)(uintptr_t)t_in, (uint64_t)(uintptr_t)t_out,
         (uint64_t)(uintptr_t)ws, (uint64_t)(uintptr_t)stream};
  for (int j = 0; j < d->l; ++j) {
    const hp_layer& w = layers[j];
    for (const hp_mat* m : {&w.wqkv, &w.wo, &w.w1, &w.w2}) {
      key.push_back((uint64_t)m->fmt);
      key.push_back((uint64_t)(uintptr_t)m->data);
      key.push_back((uint64_t)(uintptr_t)m->scale);
      key.push_back((uint64_t)(uintptr_t)m->minv);
    }
    key.push_back((uint64_t)kv[j].fmt);
    key.push_back((uint64_t)kv[j].cap);
    key.push_back((uint64_t)(uintptr_t)kv[j].k);
    key.push_back((uint64_t)(uintptr_t)kv[j].v);
    key.push_back((uint64_t)(uintptr_t)kv[j].k_sm);
    key.push_back((uint64_t)(uintptr_t)kv[j].v_sm);
  }
}

hp_status hp_run_block(const hp_dims* d, const hp_layer* layers, const void* x, const void* t_in,
                       const hp_kv* kv, void* x_out, void* t_out, void* ws, size_t ws_bytes,
                       uint32_t flags, float* times_ms, void* stream) {
  hp_status s;
  if ((s = check_dims(d)) != HP_OK) return s;
  if (!layers || !kv || !x || !x_out || !ws || (d->n > 0 && (!t_in || !t_out)))
    return fail(HP_ERR_NULL, "NULL pointer");
  NEED_ALIGN(x, 16);
  NEED_ALIGN(x_out, 16);
  NEED_ALIGN(t_in, 16);
  NEED_ALIGN(t_out, 16);
  NEED_ALIGN(ws, 256);
  // HP_DIAGONAL with page pools: every layer's pool has the same geometry
  const bool paged = (flags & HP_DIAGONAL) && kv[0].page_rows > 0;
  for (int j = 0; j < d->l; ++j) {
    if ((s = check_layer(layers[j], d->h1, d->h2)) != HP_OK) return s;
    if ((s = check_kv(&kv[j], d->s + d->n, paged ? 2 : 0)) != HP_OK) return s;
    if (paged && (kv[j].page_rows != kv[0].page_rows || kv[j].cap != kv[0].cap ||
                  kv[j].pool_pages != kv[0].pool_pages))
      return fail(HP_ERR_SHAPE, "kv[%d]: page pools of different geometry", j);
  }
  if (paged && kv[0].cap != (int)(cdiv(d->s + d->n, kv[0].page_rows) * kv[0].page_rows))
    return fail(HP_ERR_SHAPE, "paged pools: cap must be s + n rounded up to page_rows");
  const Ws L = ws_layout(*d);
  if (ws_bytes < L.total) return fail(HP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  const bool rbr = flags & HP_ROW_BY_ROW, mb = flags & HP_MICROBATCH;
  const bool graph = (flags & HP_GRAPH) && !rbr;
  const int topk_max_t = (flags & HP_TOPK10) ? d->s + d->n : 0;
  if (topk_max_t > 4096) return fail(HP_ERR_SHAPE, "HP_TOPK10 needs s + n <= 4096");
  const bool diag = flags & HP_DIAGONAL;
  if (diag && (flags & (HP_GRAPH | HP_ROW_BY_ROW | HP_MICROBATCH)))
    return fail(HP_ERR_SHAPE, "HP_DIAGONAL takes no HP_GRAPH, HP_ROW_BY_ROW or HP_MICROBATCH");
  if (graph && !stream) return fail(HP_ERR_SHAPE, "HP_GRAPH needs a non-default stream");
  if ((s = device_check()) != HP_OK) return s;
  hipStream_t st = S(stream);
  const int nbat = d->b / d->gbs;
  const int D = d->h1 / d->heads;
  const int64_t h1 = d->h1, bh = (int64_t)d->b * d->h1, sh = (int64_t)d->s * d->h1;
  int32_t* dstep = at<int32_t>(ws, L.ctr);
  _Float16* xb = at<_Float16>(ws, L.xb);
  _Float16* T0 = at<_Float16>(ws, L.t0);
  _Float16* T1 = at<_Float16>(ws, L.t1);

  // layer j of the prefill column for requests [r0, r0 + nb): activations
  // alternate between xb and x_out so that the last layer lands in x_out
  // (cache rows of requests [c0, c0 + nb); c0 = r0 except under HP_DIAGONAL)
  auto prefill_layer = [&](int j, int64_t r0, int nb, int64_t c0) {
    const _Float16* in = (j == 0) ? (const _Float16*)x
                                  : (((d->l - j) % 2 == 0) ? (const _Float16*)x_out : xb);
    _Float16* out = ((d->l - 1 - j) % 2 == 0) ? (_Float16*)x_out : xb;
    return prefill_body(nb, d->s, d->h1, d->h2, d->heads, layers[j], in + r0 * sh,
                        kv_slice(kv[j], d->heads, D, c0), out + r0 * sh, ws, L, st);
  };
  // layer j of a decode column: T0 -> T1 -> T0 ...; cache rows at s + *dstep
  auto decode_layer = [&](int j, int64_t r0, int nb) {
    const _Float16* in = (j % 2 == 0) ? T0 : T1;
    _Float16* out = (j % 2 == 0) ? T1 : T0;
    return decode_body(nb, 1, d->h1, d->h2, d->heads, layers[j], in + r0 * h1, d->s, dstep,
                       nullptr, kv_slice(kv[j], d->heads, D, r0), out + r0 * h1, ws, L, st,
                       topk_max_t);
  };
  auto stage_in = [&](int64_t r0, int nb) {
    launch_copy_step((const _Float16*)t_in + r0 * h1, nb * h1, bh, dstep, T0 + r0 * h1, 0, st);
    return launch_ok("k_copy_step");
  };
  auto stage_out = [&](int64_t r0, int nb) {
    const _Float16* last = (d->l % 2 == 1) ? T1 : T0;
    launch_copy_step(last + r0 * h1, nb * h1, bh, dstep, (_Float16*)t_out + r0 * h1, 1, st);
    hp_status r = launch_ok("k_copy_step");
    if (r != HP_OK) return r;
    launch_add_i32(dstep, 1, st);
    return launch_ok("k_set_i32");
  };

  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (times_ms) {
    for (auto& e : ev)
      if ((s = hip_ok(hipEventCreate(&e), "hipEventCreate")) != HP_OK) return s;
    if ((s = hip_ok(hipEventRecord(ev[0], st), "hipEventRecord")) != HP_OK) {
      for (auto& e : ev) (void)hipEventDestroy(e);
      return s;
    }
  }
  auto finish = [&](hp_status r) {
    if (times_ms) {
      if (r == HP_OK) r = hip_ok(hipEventRecord(ev[2], st), "hipEventRecord");
      if (r == HP_OK) r = hip_ok(hipEventSynchronize(ev[2]), "hipEventSynchronize");
      if (r == HP_OK)
        r = hip_ok(hipEventElapsedTime(&times_ms[0], ev[0], ev[1]), "hipEventElapsedTime");
      if (r == HP_OK)
        r = hip_ok(hipEventElapsedTime(&times_ms[1], ev[1], ev[2]), "hipEventElapsedTime");
      for (auto& e : ev)
        if (e) (void)hipEventDestroy(e);
    }
    return r;
  };

  if (rbr) {
    // row-by-row ([FlexGen] section 4, computation schedule): each GPU batch
    // runs its prefill and all its decode steps before the next batch starts
    if (times_ms && (s = hip_ok(hipEventRecord(ev[1], st), "hipEventRecord")) != HP_OK)
      return finish(s);
    for (int k = 0; k < nbat; ++k) {
      const int64_t r0 = (int64_t)k * d->gbs;
      for (int j = 0; j < d->l; ++j)
        if ((s = prefill_layer(j, r0, d->gbs, r0)) != HP_OK) return finish(s);
      launch_set_i32(dstep, 0, false, st);
      for (int i = 0; i < d->n; ++i) {
        if ((s = stage_in(r0, d->gbs)) != HP_OK) return finish(s);
        for (int j = 0; j < d->l; ++j)
          if ((s = decode_layer(j, r0, d->gbs)) != HP_OK) return finish(s);
        if ((s = stage_out(r0, d->gbs)) != HP_OK) return finish(s);
      }
    }
    return finish(launch_ok("row-by-row"));
  }

  if (diag && paged) {
    // diagonal block schedule ([FlexGen] appendix A.2, Fig. 5) with every live
    // request holding only the cache pages of its current length (the page's
    // peak-memory formula).  The static schedule fixes every page on the host;
    // the table goes to the workspace before the timed region.  Per iteration:
    // the live requests' inputs and row positions are gathered (one kernel),
    // then each layer runs the starting batch's prefill and one product,
    // append and attention for all live decode requests (each at its own
    // row), and the last layer's rows go to t_out (one kernel).
    const int PR = kv[0].page_rows, ppr = kv[0].cap / PR;
    std::vector<int32_t> table;
    const int64_t need = diag_page_plan(*d, PR, kv[0].cap, &table);
    if (need > kv[0].pool_pages)
      return finish(fail(HP_ERR_CAPACITY, "page pools hold %d pages, the schedule needs %lld",
                         kv[0].pool_pages, (long long)need));
    int32_t* dpt = at<int32_t>(ws, L.pt);
    int32_t* rpos = at<int32_t>(ws, L.rpos);
    if ((size_t)d->b * ppr > (size_t)d->b * cdiv(d->s + d->n, 64))
      return finish(fail(HP_ERR_SHAPE, "page table larger than its workspace region"));
    if ((s = hip_ok(hipMemcpyAsync(dpt, table.data(), table.size() * 4, hipMemcpyHostToDevice, st),
                    "hipMemcpyAsync")) != HP_OK ||
        (s = hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize")) != HP_OK)
      return finish(s);
    if (times_ms && (s = hip_ok(hipEventRecord(ev[1], st), "hipEventRecord")) != HP_OK)
      return finish(s);
    const _Float16* last = (d->l % 2 == 1) ? T1 : T0;
    for (int it = 0; it < nbat + d->n; ++it) {
      const int dlo = std::max(0, it - d->n), dhi = std::min(it - 1, nbat - 1);
      const int M = (dhi - dlo + 1) * d->gbs;  // live decode requests
      const int64_t r0 = (int64_t)dlo * d->gbs;
      if (M > 0) {
        launch_diag_rows(t_in, T0 + r0 * h1, rpos, M, (int)r0, d->gbs, d->b, d->s, it, d->h1, 0,
                         st);
        if ((s = launch_ok("k_diag_rows")) != HP_OK) return finish(s);
      }
      for (int j = 0; j < d->l; ++j) {
        hp_kv kj = kv[j];
        kj.pages = dpt;
        if (it < nbat) {
          const int64_t p0 = (int64_t)it * d->gbs;
          const _Float16* in = (j == 0) ? (const _Float16*)x
                                        : (((d->l - j) % 2 == 0) ? (const _Float16*)x_out : xb);
          _Float16* out = ((d->l - 1 - j) % 2 == 0) ? (_Float16*)x_out : xb;
          if ((s = prefill_body(d->gbs, d->s, d->h1, d->h2, d->heads, layers[j], in + p0 * sh,
                                kv_slice(kj, d->heads, D, p0), out + p0 * sh, ws, L, st)) != HP_OK)
            return finish(s);
        }
        if (M > 0) {
          const _Float16* in = (j % 2 == 0) ? T0 : T1;
          _Float16* out = (j % 2 == 0) ? T1 : T0;
          if ((s = decode_body(M, 1, d->h1, d->h2, d->heads, layers[j], in + r0 * h1,
                               d->s + d->n - 1, nullptr, nullptr, kv_slice(kj, d->heads, D, r0),
                               out + r0 * h1, ws, L, st, topk_max_t, rpos)) != HP_OK)
            return finish(s);
        }
      }
      if (M > 0) {
        launch_diag_rows(last + r0 * h1, t_out, nullptr, M, (int)r0, d->gbs, d->b, d->s, it, d->h1,
                         1, st);
        if ((s = launch_ok("k_diag_rows")) != HP_OK) return finish(s);
      }
    }
    return finish(HP_OK);
  }

  if (diag) {
    // diagonal block schedule ([FlexGen] appendix A.2, Fig. 5): GPU batch k
    // runs step it - k in iteration it (0: prefill, 1..n: decode); each
    // iteration takes layer 0 for every batch on its diagonal, then layer 1,
    // and so on.  Batch k keeps its cache in slot k mod min(nb, n + 1) from its
    // prefill to its last step.  Prefill and decode interleave: times_ms[0]
    // is 0 and times_ms[1] the whole schedule.
    if (times_ms && (s = hip_ok(hipEventRecord(ev[1], st), "hipEventRecord")) != HP_OK)
      return finish(s);
    const int nslot = std::min(nbat, d->n + 1);
    std::vector<int> pos((size_t)nbat), slot((size_t)nbat);
    const int64_t gh = (int64_t)d->gbs * h1;
    const _Float16* last = (d->l % 2 == 1) ? T1 : T0;
    for (int it = 0; it < nbat + d->n; ++it) {
      const int dlo = std::max(0, it - d->n), dhi = std::min(it - 1, nbat - 1);  // decode cells
      const int nd = dhi - dlo + 1;
      for (int k = dlo; k <= dhi; ++k) {  // batch k at step it - k reads t_in[it - k - 1]
        pos[k - dlo] = d->s + (it - k) - 1;
        slot[k - dlo] = k % nslot;
        const _Float16* src = (const _Float16*)t_in + ((int64_t)(it - k - 1) * d->b) * h1 + k * gh;
        if ((s = hip_ok(hipMemcpyAsync(T0 + k * gh, src, gh * 2, hipMemcpyDeviceToDevice, st),
                        "hipMemcpyAsync")) != HP_OK)
          return finish(s);
      }
      for (int j = 0; j < d->l; ++j) {
        if (it < nbat &&
            (s = prefill_layer(j, (int64_t)it * d->gbs, d->gbs, (int64_t)(it % nslot) * d->gbs)) !=
                HP_OK)
          return finish(s);
        if (nd > 0) {
          const _Float16* in = (j % 2 == 0) ? T0 : T1;
          _Float16* out = (j % 2 == 0) ? T1 : T0;
          if ((s = decode_cells(d->gbs, nd, pos.data(), slot.data(), d->h1, d->h2, d->heads,
                                layers[j], in + dlo * gh, kv[j], out + dlo * gh, ws, L, st,
                                topk_max_t)) != HP_OK)
            return finish(s);
        }
      }
      for (int k = dlo; k <= dhi; ++k) {
        _Float16* dst = (_Float16*)t_out + ((int64_t)(it - k - 1) * d->b) * h1 + k * gh;
        if ((s = hip_ok(hipMemcpyAsync(dst, last + k * gh, gh * 2, hipMemcpyDeviceToDevice, st),
                        "hipMemcpyAsync")) != HP_OK)
          return finish(s);
      }
    }
    return finish(HP_OK);
  }

  // zig-zag ([FlexGen] section 4, Algorithm 1): step 0 is the prefill column;
  // within a step, layer j runs for every GPU batch before layer j + 1.  The
  // GPU batches of a layer share one launch (weights read once per step)
  // unless HP_MICROBATCH asks for one launch per batch.
  const int parts = mb ? nbat : 1, nb = mb ? d->gbs : d->b;
  for (int j = 0; j < d->l; ++j)
    for (int k = 0; k < parts; ++k)
      if ((s = prefill_layer(j, (int64_t)k * nb, nb, (int64_t)k * nb)) != HP_OK) return finish(s);
  if (times_ms && (s = hip_ok(hipEventRecord(ev[1], st), "hipEventRecord")) != HP_OK)
    return finish(s);
  if (d->n == 0) return finish(HP_OK);

  launch_set_i32(dstep, 0, false, st);
  if ((s = launch_ok("k_set_i32")) != HP_OK) return finish(s);
  auto column = [&]() -> hp_status {
    hp_status r;
    if ((r = stage_in(0, d->b)) != HP_OK) return r;
    for (int j = 0; j < d->l; ++j)
      for (int k = 0; k < parts; ++k)
        if ((r = decode_layer(j, (int64_t)k * nb, nb)) != HP_OK) return r;
    return stage_out(0, d->b);
  };
  if (!graph) {
    for (int i = 0; i < d->n; ++i)
      if ((s = column()) != HP_OK) return finish(s);
    return finish(HP_OK);
  }
  std::vector<uint64_t> key;
  graph_key(key, d, layers, kv, t_in, t_out, ws, flags, stream);
  hipGraphExec_t exec = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_graphs.find(key);
    if (it != g_graphs.end()) exec = it->second;
  }
  if (!exec) {
    if ((s = hip_ok(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal), "capture")) != HP_OK)
      return finish(s);
    const hp_status body = column();
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(st, &g);
    if (body != HP_OK) {
      if (g) (void)hipGraphDestroy(g);
      return finish(body);
    }
    if ((s = hip_ok(e, "hipStreamEndCapture")) != HP_OK) return finish(s);
    const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if ((s = hip_ok(ei, "hipGraphInstantiate")) != HP_OK) return finish(s);
    std::lock_guard<std::mutex> lk(g_mu);
    g_graphs[key] = exec;
  }
  for (int i = 0; i < d->n; ++i)
    if ((s = hip_ok(hipGraphLaunch(exec, st), "hipGraphLaunch")) != HP_OK) return finish(s);
  return finish(HP_OK);
}

int32_t hp_profile(int32_t on) {
  std::lock_guard<std::mutex> lk(g_pmu);
  if (on) {
    for (auto& r : g_prec) {
      g_pool.push_back(r.second.first);
      g_pool.push_back(r.second.second);
    }
    g_prec.clear();
  }
  g_prof = on != 0;
  return HP_OK;
}

int32_t hp_profile_read(char* buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_pmu);
  std::map<std::string, std::pair<long, double>> agg;
  for (auto& r : g_prec) {
    hipError_t e = hipEventSynchronize(r.second.second);
    if (e != hipSuccess) return hip_ok(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.second.first, r.second.second);
    if (e != hipSuccess) return hip_ok(e, "hipEventElapsedTime");
    auto& a = agg[r.first];
    a.first += 1;
    a.second += ms;
  }
  std::string out;
  char line[256];
  for (auto& kv : agg) {
    snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (buf && len) {
    const size_t n = std::min(len - 1, out.size());
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return (int32_t)agg.size();
}

int64_t hp_diagonal_pages(const hp_dims* d, int32_t page_rows) {
  if (check_dims(d) != HP_OK || page_rows < 64 || (page_rows & (page_rows - 1))) return 0;
  const int cap = (int)(cdiv(d->s + d->n, page_rows) * page_rows);
  return diag_page_plan(*d, page_rows, cap, nullptr);
}

void hp_release_graphs(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& kv : g_graphs) (void)hipGraphExecDestroy(kv.second);
  g_graphs.clear();
}

uint64_t hp_weight_bytes(const hp_dims* d, int32_t fmt) {
  if (!d) return 0;
  const uint64_t elems = (uint64_t)d->l * (4ull * d->h1 * d->h1 + 2ull * d->h1 * d->h2);
  return fmt == HP_Q4 ? elems / 2 + elems / 64 * 4 : elems * 2;
}

uint64_t hp_kv_bytes(const hp_dims* d, int32_t fmt) {
  if (!d) return 0;
  const uint64_t elems = 2ull * d->b * d->l * d->h1 * (uint64_t)(d->s + d->n);
  return fmt == HP_Q4 ? elems / 2 + elems / 64 * 4 : elems * 2;
}

}  // extern "C"
