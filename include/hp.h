/*
 * hp.h -- C ABI of the MI355X (gfx950) hot path for the FlexGen OPT-style
 * transformer layer with group-wise int4 compression.
 *
 * Sources cited below:
 *   [FlexGen]  paper notes "FlexGen: High-Throughput Generative Inference of
 *              Large Language Models with a Single GPU" (ICML 2023).
 *   [SpecPipe] article "大语言模型推理加速：SpecPipe技术解析与实践".
 *
 * Notation follows [FlexGen] (background section): b requests, prompt length
 * s, n generated tokens, hidden size h1, MLP size h2, l layers.  heads splits
 * h1 into heads of d = h1/heads channels; gbs is the GPU batch size of the
 * block schedule ([FlexGen] section 4, block size = gbs x number of GPU
 * batches).
 *
 * Conventions for every entry point:
 *  - Pointers named dev_* or documented as device memory point to device
 *    memory on the current HIP device; descriptor structs (hp_dims, hp_mat,
 *    hp_layer, hp_kv) live in host memory and are read during the call only.
 *  - The caller owns and frees all device memory.  No entry point allocates
 *    device memory except hp_run_block with HP_GRAPH (it keeps one captured
 *    graph per argument set until hp_release_graphs()).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without waiting, unless stated otherwise.
 *  - Argument errors are detected on the host before anything is enqueued:
 *    the call returns a negative hp_status and hp_last_error() describes it
 *    (thread-local text).  HP_ERR_HIP reports a HIP runtime error at launch;
 *    errors raised later by the device surface at the caller's next sync.
 *  - binary16 tensors are IEEE 754 half precision; row-major throughout.
 *  - A product's rows are summed in an order fixed by (k, n) and by which
 *    side of M = 144 rows the product falls on (M <= 144: the skinny decode
 *    kernels; M > 144: the tiled kernel, another order).  Schedules whose
 *    products stay on one side of that boundary give bitwise-equal results;
 *    across it they differ by rounding only.
 *  - The device must be gfx950 (HP_ERR_DEVICE otherwise).
 */
#ifndef HP_H_
#define HP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HP_OK = 0,
  HP_ERR_NULL = -1,      /* a required pointer is NULL */
  HP_ERR_SHAPE = -2,     /* sizes violate a documented rule */
  HP_ERR_CAPACITY = -3,  /* cache rows [pos, pos+q) do not fit in cap */
  HP_ERR_TREE = -4,      /* tree arguments out of range */
  HP_ERR_WORKSPACE = -5, /* workspace smaller than hp_workspace_bytes() */
  HP_ERR_DEVICE = -6,    /* no device, or the device is not gfx950 */
  HP_ERR_HIP = -7        /* a HIP runtime call failed */
} hp_status;

/* Storage formats. */
enum { HP_F16 = 0, HP_Q4 = 1 };

/*
 * Group-wise asymmetric int4 ([FlexGen] section 5, group-wise quantization):
 * a group is 64 consecutive elements along one dimension; each element is
 * coded as c = round((x - min) / (max - min) * 15) and read back as
 * fp16(c * scale + min).  Exact definition used here (the page gives the
 * real-number formula only):
 *   - x is the fp16 value as binary32, with -0 taken as +0;
 *   - min/max skip NaN (IEEE minNum/maxNum); r = max - min in binary32;
 *   - if !(r > 0): every code 0, scale = +0, min = fp16(min) (+0 if no finite
 *     element);
 *   - else scale = fp16(r / 15), min = fp16(min), and
 *     c = clamp(rint(((x - min) / r) * 15), 0, 15) in binary32 with
 *     correctly rounded division and round-half-to-even rint (NaN -> 0);
 *   - dequantised value: fp16(c * scale + min) with a single rounding.
 * Generic ("row") layout, used for the KV cache and hp_quantize_g64:
 *   codes u8[rows][cols/2], byte j of a group = c[2j] | c[2j+1] << 4;
 *   sm = half2 {scale, min} [rows][cols/64].
 */

/*
 * Weight matrix w in[h_in = k][h_out = n] of the product x·w ([FlexGen]
 * background section).  Weights are grouped along the output-channel
 * dimension ([FlexGen] section 5): a group is w[kk][64 g .. 64 g + 63].
 * Stored in the GEMM layout produced by hp_pack_weight_*:
 *   HP_F16: data = half tiles[k/128][n/16][4][64][8]: tile (kb, nb), k-step
 *           j, lane L (0..63) holds the 8 inputs kk = 128 kb + 32 j +
 *           8 (L / 16) + e, e = 0..7, of output column n = 16 nb + L % 16
 *           (the MFMA operand fragments of one k-step are one contiguous
 *           1 KB; the tiles of one k-block are adjacent).
 *   HP_Q4:  data = u8 tiles[n/16][k/128][64][16]: tile (nb, kb), lane L
 *           (0..63) holds the 32 codes of output column n = 16 nb + L % 16
 *           at inputs kk = 128 kb + 32 (L / 16) + 0..31, as 4 dwords; dword
 *           j holds kk-offsets 8 j + e, e = 0..7, with offset e in nibble
 *           (e even ? e / 2 : 4 + e / 2) (bits 4*nibble .. 4*nibble+3);
 *           scale = half [n/64][k], minv = half [n/64][k] (per group).
 *   Requires k % 128 == 0 and n % 64 == 0.
 */
typedef struct {
  int32_t fmt;       /* HP_F16 or HP_Q4 */
  int32_t k, n;      /* h_in, h_out */
  const void* data;  /* device */
  const void* scale; /* device, HP_Q4 only (else NULL) */
  const void* minv;  /* device, HP_Q4 only (else NULL) */
} hp_mat;

/* One layer.  wqkv is [h1 -> 3 h1] with output columns Q | K | V (the
 * concatenation of w_Q, w_K, w_V); wo [h1 -> h1]; w1 [h1 -> h2];
 * w2 [h2 -> h1].  All four use the same fmt. */
typedef struct {
  hp_mat wqkv, wo, w1, w2;
} hp_layer;

/* One layer's KV cache ([FlexGen] decode equations: rows grow by Concat;
 * section 5: KV grouped along the hidden dimension).  Head-major:
 *   HP_F16: k, v = half [b][heads][cap][d];  k_sm = v_sm = NULL.
 *   HP_Q4:  k, v = u8 codes [b][heads][cap][d/2] (generic row layout, one
 *           row = one token of one head, groups of 64 channels),
 *           k_sm, v_sm = half2 {scale, min} [b][heads][cap][d/64].
 * All pointers are device memory; b is the request count of the call.
 *
 * Paged caches (page_rows > 0): k, v, k_sm, v_sm are pools of pool_pages
 * pages, page p holding page_rows rows of every head, [p][heads][page_rows]
 * [row] in the layouts above; row j of request r, head h is row
 * j % page_rows of page pages[r * (cap / page_rows) + j / page_rows]
 * (device int32 [b][cap / page_rows]; entries outside [0, pool_pages) are
 * clamped into it).  cap is then the logical rows per request, a multiple
 * of page_rows; page_rows is a power of two, at least 64.  hp_kv_append,
 * hp_decode_attention / hp_decode_attention_ragged with q < 16 and
 * hp_topk_attention take paged caches; the other cache calls return
 * HP_ERR_SHAPE for them.  Under
 * HP_DIAGONAL, hp_run_block assigns the pages itself (pages = NULL; see
 * HP_DIAGONAL).  Contiguous caches: pages = NULL, page_rows = pool_pages
 * = 0. */
typedef struct {
  int32_t fmt, cap;
  void *k, *v, *k_sm, *v_sm;
  const int32_t* pages;
  int32_t page_rows, pool_pages;
} hp_kv;

typedef struct {
  int32_t b, s, n, h1, h2, l, heads, gbs;
} hp_dims;
/* Shape rules checked by every layer/block entry point: all sizes > 0;
 * h1 % heads == 0 with d = h1/heads in {64, 128}; h1 % 128 == 0;
 * h2 % 128 == 0; b % gbs == 0; weights and cache formats consistent with
 * the dims. */

/* ------------------------------------------------------------ diagnostics */
const char* hp_last_error(void);
/* 0 if the current device is gfx950 and usable, else HP_ERR_DEVICE. */
hp_status hp_device_check(void);

/* ---------------------------------------------------------- compression */
/* [FlexGen] section 5.  x: device half[rows][cols], groups of 64 along cols
 * (cols % 64 == 0, rows >= 0).  Writes codes (device u8[rows][cols/2]) and
 * sm (device half2[rows][cols/64]) in the generic layout above. */
hp_status hp_quantize_g64(const void* x, int64_t rows, int64_t cols, void* codes, void* sm,
                          void* stream);

/* [FlexGen] section 5 (converted back to FP16 before computation).
 * y: device half[rows][cols] = fp16(c * scale + min), single rounding. */
hp_status hp_dequantize_g64(const void* codes, const void* sm, int64_t rows, int64_t cols,
                            void* y, void* stream);

/* Rearranges a quantised weight w[k][n] (generic layout: codes u8[k][n/2],
 * sm half2[k][n/64], groups along n) into the HP_Q4 GEMM layout (packed
 * tiles, scale, minv; see hp_mat).  Codes are moved, never recomputed. */
hp_status hp_pack_weight_q4(const void* codes, const void* sm, int32_t k, int32_t n,
                            void* packed, void* scale, void* minv, void* stream);

/* fp16 weight w[k][n] (device) -> the HP_F16 GEMM layout (see hp_mat;
 * k * n halves, 16-byte aligned).  Requires k % 128 == 0, n % 64 == 0. */
hp_status hp_pack_weight_f16(const void* w, int32_t k, int32_t n, void* wt, void* stream);

/* ---------------------------------------------------------- layer stages */
/* y[M][n] = fp16(act(x·w) + res): x device half [M][k] (row stride ldx),
 * w in GEMM layout, res device half [M][n] (row stride ldr) or NULL,
 * act = ReLU if relu != 0.  y row stride ldy.  Sums in binary32 over k in an
 * order fixed by (k, n).  [FlexGen] background section: every projection
 * and MLP product of the layer is such a product.  ws: device scratch of at
 * least hp_gemm_workspace_bytes(M, k, n, w->fmt) bytes (may be NULL when that
 * is 0): split-k partial sums when M <= 144, the FP16 expansion of an int4
 * weight when M > 144. */
size_t hp_gemm_workspace_bytes(int64_t M, int32_t k, int32_t n, int32_t fmt);
hp_status hp_gemm(const void* x, int64_t ldx, const hp_mat* w, int64_t M, const void* res,
                  int64_t ldr, int32_t relu, void* y, int64_t ldy, void* ws, size_t ws_bytes,
                  void* stream);

/* hp_gemm for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same product, kernels and results as hp_gemm
 * (bit for bit), with the split-k partial sums in a static device array of
 * 64 MiB that the library holds on each GPU it runs on until the process
 * ends.  Nothing is allocated.  Takes 1 <= M <= 144 rows (the decode-step
 * products; M = 0 is a no-op); a taller M, or a product whose partials need
 * more than 64 MiB (hp_gemm_workspace_bytes), returns HP_ERR_SHAPE or
 * HP_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on a GPU (concurrent streams or
 * host threads) race and must be serialised by the caller; each call
 * overwrites every partial it reads, so nothing needs clearing. */
hp_status hp_gemm_noalloc(const void* x, int64_t ldx, const hp_mat* w, int64_t M,
                          const void* res, int64_t ldr, int32_t relu, void* y, int64_t ldy,
                          void* stream);

/* [FlexGen] decode equations (Concat) and section 5 (KV grouped along the
 * hidden dimension): for each request r < b and new token i < q, copies (or
 * quantises) the K and V rows of token i into cache rows pos + i.
 * qkv: device half [b][q][3 h1] with K at columns [h1, 2 h1) and V at
 * [2 h1, 3 h1).  Requires pos + q <= kv->cap. */
hp_status hp_kv_append(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                       int32_t pos, const hp_kv* kv, void* stream);

/* hp_kv_append with a row position per request (requests at different
 * lengths, as in the diagonal block schedule): request r's token i goes to
 * row rpos[r] + i, rpos: device int32 [b], each clamped to [0, max_pos].
 * Requires max_pos + q <= kv->cap. */
hp_status hp_kv_append_ragged(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                              const int32_t* rpos, int32_t max_pos, const hp_kv* kv,
                              void* stream);

/* Causal prefill attention over the fresh K/V ([FlexGen] prefill equations;
 * causal mask: query i sees keys 0..i).  qkv: device half [b][s][3 h1]
 * (Q | K | V columns); out: device half [b][s][h1]. */
hp_status hp_prefill_attention(int32_t b, int32_t s, int32_t h1, int32_t heads, const void* qkv,
                               void* out, void* stream);

/* Decode attention over the cache ([FlexGen] decode equations; [SpecPipe]
 * 2.2.1-2.2.2 for tree masks).  For request r and new token i < q (its K/V
 * already appended at row pos + i), query i reads, through the stored
 * format, cache rows [0, pos) and each row pos + u with bit u of
 * masks[r][i] set; masks == NULL means a chain (rows pos .. pos + i).
 * q in [1, 64].  qkv: device half [b][q][3 h1] (the query is read from
 * columns [0, h1)); masks: device uint64 [b][q] or NULL; out: device half
 * [b][q][h1].  Requires pos + q <= kv->cap. */
hp_status hp_decode_attention(int32_t b, int32_t q, int32_t h1, int32_t heads, const void* qkv,
                              int32_t pos, const uint64_t* masks, const hp_kv* kv, void* out,
                              void* stream);

/* hp_decode_attention with a prefix length per request, as after tree
 * pruning (hp_tree_prune): query i of request r reads rows [0, P) and each
 * row P + u with bit u of masks[r][i] set (masks == NULL: a chain, rows
 * P .. P + i), P = prefix[r] (device int32 [b]) clamped to [0, max_prefix].
 * Requires max_prefix + q <= kv->cap; other arguments as in
 * hp_decode_attention. */
hp_status hp_decode_attention_ragged(int32_t b, int32_t q, int32_t h1, int32_t heads,
                                     const void* qkv, const int32_t* prefix, int32_t max_prefix,
                                     const uint64_t* masks, const hp_kv* kv, void* out,
                                     void* stream);

/* Top-K sparse decode attention ([FlexGen] section 5, sparse attention): for
 * request r's new token (its K/V already appended at row pos), the scores
 * q . k_j over cache rows j in [0, pos] are formed through the stored format,
 * the K largest are kept (ties to the lower row), the other rows are dropped
 * and the output is the attention over the kept rows only (softmax over
 * them; only their V rows are read).  K = topk (at most pos + 1), or
 * ceil((pos + 1) / 10) when topk == 0.  qkv: device half [b][3 h1] (query in
 * columns [0, h1)); out: device half [b][h1]; idx: device int32
 * [b][heads][K] receiving the kept rows in ascending order, or NULL.
 * Contiguous or paged caches (see hp_kv).  Requires pos + 1 <= min(kv->cap,
 * 4096). */
hp_status hp_topk_attention(int32_t b, int32_t h1, int32_t heads, const void* qkv, int32_t pos,
                            int32_t topk, const hp_kv* kv, void* out, int32_t* idx, void* stream);

/* [SpecPipe] 2.2.1 (tree mask M): builds masks[r][i] (bit u set iff token u
 * is token i or one of its ancestors) from a BFS parent array per request:
 * parent: device int32 [b][q], parent[r][0] == -1 and
 * 0 <= parent[r][i] < i for i > 0.  err: device int32, set to the number of
 * parent entries that break these rules (their masks hold only the token
 * itself).  q in [1, 64]. */
hp_status hp_tree_masks(int32_t b, int32_t q, const int32_t* parent, uint64_t* masks,
                        int32_t* err, void* stream);

/* [SpecPipe] 2.2.1 sub-tree pruning (Fig. 5-b) and 2.2.2 (Fig. 8): when
 * token u = verified[r] of request r's BFS tree of q tokens (cache rows
 * pos .. pos + q - 1 after a prefix of pos rows) is verified, the tree keeps
 * u and its descendants (column u of the mask matrix), in BFS order, and u
 * becomes its root; the rows of the verified path above u (the root down to
 * u's parent) stay in the cache as committed prefix.  parent: device int32
 * [b][q] (rules of hp_tree_masks); verified: device int32 [b].  Outputs
 * (device int32):
 *   prefix[r] = pos + depth, depth = number of u's ancestors: the new
 *               prefix length (the path rows are committed);
 *   kept[r]   = size of the new tree (u's subtree, u included);
 *   src[r][j] = for j < depth + kept[r], the old tree index of the token
 *               whose cache row goes to row pos + j: the path (root first),
 *               then the new tree's tokens in order; -1 beyond;
 *   new_parent[r][t] = for t < kept[r], the new index of token t's parent
 *               (-1 for u, at t = 0); entries t >= kept[r] are filler leaves
 *               (the last kept token's parent, or 0 when u is alone), so
 *               new_parent is again a valid BFS parent array.
 * Token t of the new tree is old token src[r][depth + t]; after
 * hp_kv_compact its K/V rows sit at prefix[r] + t.  A request with an invalid
 * parent array or verified index outside [0, q) keeps nothing (prefix = pos,
 * kept 0, new_parent a star, src -1); err (device int32, or NULL) is set to
 * the number of such requests.  q in [1, 64]; one kernel launch (one wave
 * per request). */
hp_status hp_tree_prune(int32_t b, int32_t q, const int32_t* parent, const int32_t* verified,
                        int32_t pos, int32_t* new_parent, int32_t* src, int32_t* prefix,
                        int32_t* kept, int32_t* err, void* stream);

/* Moves one layer's surviving rows into place after hp_tree_prune: for
 * request r and every head, cache row pos + j, j < prefix[r] - pos + kept[r],
 * takes the K and V rows (codes and scale/min, or fp16) of row
 * pos + src[r][j].  Rows [0, pos) and the rows after the moved ones (up to
 * pos + q) are not touched.  src, prefix, kept: device int32 as written by
 * hp_tree_prune (a count outside [0, q] is clamped to it).  Requires
 * pos + q <= kv->cap. */
hp_status hp_kv_compact(int32_t b, int32_t q, int32_t h1, int32_t heads, int32_t pos,
                        const int32_t* src, const int32_t* prefix, const int32_t* kept,
                        const hp_kv* kv, void* stream);

/* ------------------------------------------------------------- layers */
/* Workspace for hp_layer_prefill / hp_layer_decode / hp_run_block with these
 * dims (bytes of device memory, 256-byte aligned by the caller). */
size_t hp_workspace_bytes(const hp_dims* d);

/* One layer, prefill ([FlexGen] background section, prefill equations):
 * x device half [b][s][h1] -> x_out device half [b][s][h1]; writes cache
 * rows [0, s) of every request (d->b requests).  Requires s <= kv->cap. */
hp_status hp_layer_prefill(const hp_dims* d, const hp_layer* w, const void* x, const hp_kv* kv,
                           void* x_out, void* ws, size_t ws_bytes, void* stream);

/* One layer, decode ([FlexGen] decode equations): t device half
 * [b][q][h1] at cache rows [pos, pos + q) -> t_out device half [b][q][h1].
 * masks as in hp_decode_attention (NULL: chain; q == 1 is the plain
 * decode step).  Requires pos + q <= kv->cap and q <= 64. */
hp_status hp_layer_decode(const hp_dims* d, const hp_layer* w, const void* t, int32_t pos,
                          int32_t q, const uint64_t* masks, const hp_kv* kv, void* t_out,
                          void* ws, size_t ws_bytes, void* stream);

/* Diagnostics for teacher-forced checks: the fp16 tensors a layer stores
 * between its stages ([FlexGen] background section: Q/K/V, the attention
 * output, x_Out and the MLP hidden relu(x_Out w_1); section 5: K/V are
 * quantised from the stored fp16 rows).  While a capture is set on the
 * calling thread, every hp_layer_prefill and hp_layer_decode call on that
 * thread copies them, after the layer, into the given device buffers
 * (M = b s rows for prefill, b q for decode; any pointer may be NULL):
 *   qkv    half [M][3 h1]  (Q | K | V, the rows appended to the cache),
 *   attn   half [M][h1]    (softmax(Q K^T / sqrt(d)) V),
 *   x_out  half [M][h1]    (attn w_O + x),
 *   hidden half [M][h2]    (relu(x_out w_1)).
 * The buffers must hold M rows; the copies are enqueued on the layer's
 * stream.  hp_debug_set_capture(NULL) turns capturing off.  hp_run_block
 * never captures. */
typedef struct {
  void* qkv;
  void* attn;
  void* x_out;
  void* hidden;
} hp_capture;
hp_status hp_debug_set_capture(const hp_capture* c);

/* --------------------------------------------------------- block schedule */
enum {
  HP_GRAPH = 1,      /* capture one decode column as a hipGraph, replay it n times */
  HP_ROW_BY_ROW = 2, /* row-by-row order: each GPU batch runs all steps alone */
  HP_MICROBATCH = 4, /* zig-zag with one launch per GPU batch (gbs rows)
                        instead of one launch per block */
  HP_TOPK10 = 8,     /* decode columns use Top-K sparse attention keeping
                        ceil(T / 10) of the T visible rows ([FlexGen] section 5,
                        sparse attention; see hp_topk_attention); s + n <= 4096 */
  HP_DIAGONAL = 16   /* diagonal block schedule ([FlexGen] appendix A.2, Fig. 5):
                        GPU batch k runs step it - k of iteration it (0 = its
                        prefill), layer-major over the batches of each
                        iteration; results equal the zig-zag block's bit for
                        bit when each product of the two schedules falls on
                        the same side of M = 144 rows (always for b <= 144),
                        within rounding otherwise.  Eager launches: not with
                        HP_GRAPH, HP_ROW_BY_ROW or HP_MICROBATCH
                        (HP_ERR_SHAPE).  times_ms[0] = 0, times_ms[1] = the
                        whole schedule.  Two cache modes, set by kv[j]:
                        - contiguous (page_rows 0): batch k keeps its cache
                          in slot k mod min(b / gbs, n + 1), so kv[j] needs
                          only that many GPU batches of requests (cap >=
                          s + n); append and attention run per batch;
                        - paged (page_rows > 0, pages NULL): kv[j] is a pool
                          of pool_pages pages and every live request holds
                          only the pages its current length needs (freed
                          after its last step), so the pool follows the
                          page's peak-memory formula instead of b (s + n)
                          rows; hp_diagonal_pages() gives the pages needed.
                          One product, append and attention per layer and
                          iteration for all live batches (with HP_TOPK10,
                          Top-K attention over each request's own rows). */
};

/* [FlexGen] section 4, Algorithm 1: zig-zag block schedule over one block of
 * d->b = gbs x (b/gbs) requests.  Step 0 is the prefill column over x
 * (device half [b][s][h1]); steps 1..n are decode columns fed the given
 * embeddings t_in (device half [n][b][h1]; the pages define no token
 * sampling).  Within a step, layer j runs for the whole block before layer
 * j + 1, so each layer's weights are read once per step for the block.
 * layers: host array of d->l hp_layer; kv: host array of d->l hp_kv with
 * cap >= s + n.  Outputs: x_out device half [b][s][h1] (last layer, prefill)
 * and t_out device half [n][b][h1] (last layer, each decode step).
 * times_ms: NULL, or a host float[2] that receives the prefill and decode
 * durations measured with HIP events on `stream` (the call then waits for
 * the stream before returning). */
hp_status hp_run_block(const hp_dims* d, const hp_layer* layers, const void* x, const void* t_in,
                       const hp_kv* kv, void* x_out, void* t_out, void* ws, size_t ws_bytes,
                       uint32_t flags, float* times_ms, void* stream);

/* [FlexGen] appendix A.2 (diagonal block schedule, peak memory): the number of
 * cache pages of page_rows rows (per request, all heads; a power of two, at
 * least 64)
 * that HP_DIAGONAL with paged caches holds at its peak for these dims: live
 * requests hold ceil(current length / page_rows) pages each.  0 for invalid
 * dims or page_rows. */
int64_t hp_diagonal_pages(const hp_dims* d, int32_t page_rows);

/* Drops every captured graph (device memory of graph execs is released). */
void hp_release_graphs(void);

/* ------------------------------------------------------------ profiling */
/* Diagnostics.  hp_profile(1) clears earlier records and makes every later
 * kernel launch of the library record a start/stop HIP event pair on its own
 * stream (launches inside a graph capture are not recorded); hp_profile(0)
 * stops recording.  hp_profile_read() waits for the recorded events and
 * writes one line "kernel launches total_ms" per kernel name into buf
 * (NUL-terminated, truncated to len bytes); it returns the number of lines,
 * or a negative hp_status. */
int32_t hp_profile(int32_t on);
int32_t hp_profile_read(char* buf, size_t len);

/* ---------------------------------------------------- achievable peaks */
/* Measurement probes, not part of the layer: the rates this GPU attains on
 * the two resources the kernels are bound by, the reference for their
 * fractions beside the published peaks.  hp_peak_read streams `bytes` bytes
 * of the device buffer x once (16-byte non-temporal loads; x and bytes
 * multiples of 16) over `workgroups` workgroups of 256 threads.
 * hp_peak_mfma runs `iters` rounds of 16 independent
 * v_mfma_f32_16x16x32_f16 (16 x 16 x 32 fp16 products, 16384 flop each) in
 * each of the 8 waves of `workgroups` workgroups of 512 threads (operand
 * values arbitrary): 8 * 16 * iters * 16384 flop per workgroup.  sink:
 * device uint32, at least workgroups (read) or 8 * workgroups (mfma) words,
 * contents meaningless.  Both enqueue on `stream` (time them with events)
 * and return HP_ERR_NULL / HP_ERR_SHAPE for bad arguments. */
hp_status hp_peak_read(const void* x, uint64_t bytes, int32_t workgroups, uint32_t* sink,
                       void* stream);
hp_status hp_peak_mfma(int32_t iters, int32_t workgroups, uint32_t* sink, void* stream);

/* ------------------------------------------------------------ sizes */
/* [FlexGen] background section (memory bottleneck analysis): weight bytes
 * l(8 h1^2 + 4 h1 h2) in fp16, and peak KV bytes 4 b l h1 (s + n) in fp16;
 * fmt HP_Q4 gives the packed sizes (codes plus fp16 scale/min per group). */
uint64_t hp_weight_bytes(const hp_dims* d, int32_t fmt);
uint64_t hp_kv_bytes(const hp_dims* d, int32_t fmt);

#ifdef __cplusplus
}
#endif
#endif /* HP_H_ */
