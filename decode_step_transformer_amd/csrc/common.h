// Internal helpers shared by the HIP sources of libhp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/hp.h"

namespace hp {

// Thread-local error text behind hp_last_error().
hp_status fail(hp_status st, const char* fmt, ...);
// Checks a HIP runtime result; sets the error text on failure.
hp_status hip_ok(hipError_t e, const char* what);
// Checks the last launch on this thread.
hp_status launch_ok(const char* kernel);

inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Per-kernel event timing (hp_profile): while enabled, a Prof object records
// a start event on construction and a stop event on destruction, on the
// launch stream, unless that stream is being captured into a graph.
struct Prof {
  Prof(const char* tag, hipStream_t st);
  ~Prof();
  const char* tag;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
};

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- launchers implemented in the .hip files (all enqueue on `st`) ----
void launch_quantize_g64(const void* x, int64_t rows, int64_t cols, void* codes, void* sm,
                         hipStream_t st);
void launch_dequantize_g64(const void* codes, const void* sm, int64_t rows, int64_t cols, void* y,
                           hipStream_t st);
void launch_pack_q4(const void* codes, const void* sm, int32_t k, int32_t n, void* packed,
                    void* scale, void* minv, hipStream_t st);
void launch_pack_f16(const void* w, int32_t k, int32_t n, void* wt, hipStream_t st);

// GEMM: y = act(x·w) + res (see hp_gemm).  ws holds split-K partials.
size_t gemm_ws_bytes(int64_t M, int32_t k, int32_t n, int32_t fmt);
hp_status launch_gemm(const void* x, int64_t ldx, const hp_mat& w, int64_t M, const void* res,
                      int64_t ldr, bool relu, void* y, int64_t ldy, void* ws, hipStream_t st);

// Largest M run as a skinny product (one row tile, split k); taller products
// run on the tiled kernel.
constexpr int64_t kSkinnyM = 144;
// Size of the static scratch behind hp_gemm_noalloc (split-k partials of
// skinny products: 63.7 MB at the largest, the 175B QKV product at M = 144).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress).
hp_status static_scratch(void** ptr);

// Skinny int4 product (1 <= M <= 144) on the 8-wave decode kernel; with
// splits > 1 the k-range is split, fp32 partials go to `partials` (the
// kernel's tile-major layout, gemm_ws_bytes of them) and a second kernel adds
// them in split order.
hp_status launch_gemm_dq(const void* x, int64_t ldx, const hp_mat& w, int64_t M, const void* res,
                         int64_t ldr, bool relu, void* y, int64_t ldy, int splits, float* partials,
                         hipStream_t st);

// fp16 tiled product for tall M and the int4 -> fp16 weight expansion that
// feeds it.  ldw == 0: wt is in the fragment-major HP_F16 layout; else wt =
// [n][k] fp16 rows of stride ldw (the expansion's output).
hp_status launch_gemm16(const void* x, int64_t ldx, const void* wt, int64_t ldw, int k, int n,
                        int64_t M, const void* res, int64_t ldr, bool relu, void* y, int64_t ldy,
                        hipStream_t st);
// int4 weight -> fp16 wt[n][k] (row stride ldw) for the tall products.
hp_status launch_expand_q4(const hp_mat& w, void* wt, int64_t ldw, hipStream_t st);

// Row stride (elements of 2 bytes) for an internal [rows][n] fp16 buffer:
// rows whose byte length is a multiple of 16 KB put the same column of
// consecutive rows on the same HBM channels, which cut the tall GEMM to
// three quarters of its speed when such a buffer is its input (measured at
// n = 49152); 128 bytes more per row break the alias.
inline int64_t pad_ld(int64_t n) { return n % 8192 == 0 ? n + 64 : n; }

// KV append / attention.  `dpos` (device int32, may be NULL): when set, the
// kernels read pos from it (plus pos as an offset), so a captured graph can
// be replayed at advancing positions.
// rpos (device int32 [b], may be NULL): per-request first rows, each clamped
// to [0, pos]; then dpos is ignored.  Paged caches (kv.page_rows > 0) go
// through kv.pages.
void launch_kv_append(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                      int32_t pos, const int32_t* dpos, const int32_t* rpos, const hp_kv& kv,
                      hipStream_t st);
void launch_prefill_attention(int32_t b, int32_t s, int32_t h1, int32_t heads, const void* qkv,
                              void* out, hipStream_t st);
// plen (device int32 [b], may be NULL): per-request prefix lengths, each
// clamped to [0, pos]; then dpos is ignored.
void launch_decode_attention(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                             int32_t pos, const int32_t* dpos, const int32_t* plen,
                             const uint64_t* masks, const hp_kv& kv, void* out, hipStream_t st);
// Top-K sparse decode attention (one query per request); visible rows
// [0, pos + *dpos + 1), or [0, min(rpos[r], pos) + 1) for request r when rpos
// is given, with max_t bounding that count (<= 4096); topk = 0 keeps
// ceil(T / 10).  Contiguous or paged caches.  Returns HP_ERR_SHAPE if max_t is
// out of range.
hp_status launch_topk_attention(int32_t b, int32_t h1, int32_t heads, const void* qkv, int32_t pos,
                                const int32_t* dpos, int32_t max_t, int32_t topk, const hp_kv& kv,
                                void* out, int32_t* idx, hipStream_t st,
                                const int32_t* rpos = nullptr);
void launch_tree_masks(int32_t b, int32_t q, const int32_t* parent, uint64_t* masks, int32_t* err,
                       hipStream_t st);
void launch_tree_prune(int32_t b, int32_t q, int32_t pos, const int32_t* parent,
                       const int32_t* verified, int32_t* new_parent, int32_t* src,
                       int32_t* prefix, int32_t* kept, int32_t* err, hipStream_t st);
void launch_kv_compact(int32_t b, int32_t q, int32_t heads, int32_t d, int32_t pos,
                       const int32_t* src, const int32_t* prefix, const int32_t* kept,
                       const hp_kv& kv, hipStream_t st);

// Small utility kernels used by the block runner.
void launch_copy_step(const void* src, int64_t count_elems, int64_t stride_elems,
                      const int32_t* dstep, void* dst, int direction, hipStream_t st);
void launch_add_i32(int32_t* p, int32_t v, hipStream_t st);

}  // namespace hp
