// Group-wise int4 quantisation ([FlexGen] paper notes, section 5,
// group-wise quantization) and the weight packers for the GEMM layout.
//
// quantize: one group of 64 fp16 values = 128 bytes is read by 8 lanes with
// 16-byte loads (a wave covers 8 groups = 1 KB, fully coalesced); min/max
// are reduced over the 8 lanes with xor shuffles; each lane then codes its
// 8 elements and writes one dword of packed nibbles.  HBM-bound: 128 B in,
// 36 B out per group.
#include "common.h"
#include "quant_dev.h"

namespace hp {

// Each lane codes QU groups whose loads are all issued before the first is
// used: with one 16-byte load per lane in flight, even a full CU (32 waves)
// holds only 32 KB of requests, too few to cover HBM latency.
constexpr int QU = 4;

__global__ __launch_bounds__(256) void k_quantize_g64(const uint4* __restrict__ x, int64_t groups,
                                                      uint32_t* __restrict__ codes,
                                                      uint32_t* __restrict__ sm) {
  const int sub = threadIdx.x & 7;
  // block: QU runs of 32 groups; wave w takes groups 8 w .. 8 w + 7 of each run
  const int64_t g0 = (int64_t)blockIdx.x * (32 * QU) + (threadIdx.x >> 3);
  uint4 raw[QU];
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const int64_t g = g0 + 32 * u;
    if (g < groups) raw[u] = stream_load16(x + g * 8 + sub);
  }
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const int64_t g = g0 + 32 * u;
    if (g < groups) {  // the same for the 8 lanes of a group
      uint32_t smw;
      const uint32_t word = quant_group8(raw[u], smw);
      __builtin_nontemporal_store(word, codes + g * 8 + sub);  // streamed out
      if (sub == 0) sm[g] = smw;
    }
  }
}

__global__ __launch_bounds__(256) void k_dequantize_g64(const uint32_t* __restrict__ codes,
                                                        const uint32_t* __restrict__ sm,
                                                        int64_t words, uint4* __restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) {
    const uint32_t w = codes[i];
    const uint32_t s = sm[i >> 3];
    const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(s & 0xffff));
    const _Float16 mn = __builtin_bit_cast(_Float16, (uint16_t)(s >> 16));
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const _Float16 c0 = (_Float16)(float)((w >> (8 * p)) & 15);
      const _Float16 c1 = (_Float16)(float)((w >> (8 * p + 4)) & 15);
      const _Float16 y0 = __builtin_fmaf16(c0, sc, mn);
      const _Float16 y1 = __builtin_fmaf16(c1, sc, mn);
      out[p] = (uint32_t)__builtin_bit_cast(uint16_t, y0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
    }
    y[i] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// One thread per output dword of the packed q4 weight layout (see hp_mat).
__global__ __launch_bounds__(256) void k_pack_q4(const uint8_t* __restrict__ codes, int32_t k,
                                                 int32_t n, uint32_t* __restrict__ packed) {
  const int64_t total = (int64_t)n * k / 8;
  const int KB = k / 128;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int j = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t tile = idx >> 8;
    const int kb = (int)(tile % KB);
    const int nb = (int)(tile / KB);
    const int col = 16 * nb + (lane & 15);
    const int k0 = 128 * kb + 32 * (lane >> 4) + 8 * j;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint8_t byte = codes[(int64_t)(k0 + e) * (n / 2) + col / 2];
      const uint32_t c = (col & 1) ? (byte >> 4) : (byte & 15);
      const int nib = (e & 1) ? 4 + (e >> 1) : (e >> 1);
      word |= c << (4 * nib);
    }
    packed[idx] = word;
  }
}

__global__ __launch_bounds__(256) void k_pack_sm(const uint32_t* __restrict__ sm, int32_t k,
                                                 int32_t n, uint16_t* __restrict__ scale,
                                                 uint16_t* __restrict__ minv) {
  const int G = n / 64;
  const int64_t total = (int64_t)k * G;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t g = idx / k, kk = idx % k;
    const uint32_t v = sm[kk * G + g];
    scale[idx] = (uint16_t)(v & 0xffff);
    minv[idx] = (uint16_t)(v >> 16);
  }
}

// fp16 w[k][n] -> the fragment-major HP_F16 layout: tile (kb, nb) of 16
// output columns x 128 inputs is 4 KB contiguous at (kb (n / 16) + nb) 4 KB,
// [j][lane][8] halves, lane L holding column 16 nb + L % 16 at inputs
// 128 kb + 32 j + 8 (L / 16) + e (exactly one MFMA operand fragment per
// k-step j; the tiles of one k-block are adjacent).  64 x 64 tiles of w pass
// through LDS; each thread writes 8 consecutive inputs of one column (16 B).
__global__ __launch_bounds__(256) void k_pack_f16(const uint16_t* __restrict__ w, int32_t k,
                                                  int32_t n, uint16_t* __restrict__ wt) {
  __shared__ uint16_t tile[64][65];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    tile[r][c] = w[(int64_t)(k0 + r) * n + n0 + c];
  }
  __syncthreads();
  const int64_t NB = n / 16;
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int c = i / 8, k8 = (i % 8) * 8;  // column n0 + c, inputs k0 + k8 .. + 7
    const int nn = n0 + c, kk = k0 + k8;
    const int64_t off = (((int64_t)(kk / 128) * NB + nn / 16) * 4 + (kk % 128) / 32) * 512 +
                        ((nn % 16) + 16 * ((kk % 32) / 8)) * 8;
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)tile[k8 + 2 * e][c] | ((uint32_t)tile[k8 + 2 * e + 1][c] << 16);
    *(uint4*)(wt + off) = uint4{v[0], v[1], v[2], v[3]};
  }
}

static int grid_for(int64_t items, int per_block) {
  int64_t g = cdiv(items, per_block);
  if (g > 256 * 64) g = 256 * 64;
  return (int)(g < 1 ? 1 : g);
}

void launch_quantize_g64(const void* x, int64_t rows, int64_t cols, void* codes, void* sm,
                         hipStream_t st) {
  const int64_t groups = rows * (cols / 64);
  if (groups == 0) return;
  Prof prof("quantize_g64", st);
  hipLaunchKernelGGL(k_quantize_g64, dim3((unsigned)cdiv(groups, 32 * QU)), dim3(256), 0, st,
                     (const uint4*)x, groups, (uint32_t*)codes, (uint32_t*)sm);
}

void launch_dequantize_g64(const void* codes, const void* sm, int64_t rows, int64_t cols, void* y,
                           hipStream_t st) {
  const int64_t words = rows * cols / 8;
  if (words == 0) return;
  Prof prof("dequantize_g64", st);
  hipLaunchKernelGGL(k_dequantize_g64, dim3(grid_for(words, 256)), dim3(256), 0, st,
                     (const uint32_t*)codes, (const uint32_t*)sm, words, (uint4*)y);
}

void launch_pack_q4(const void* codes, const void* sm, int32_t k, int32_t n, void* packed,
                    void* scale, void* minv, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_q4, dim3(grid_for((int64_t)n * k / 8, 256)), dim3(256), 0, st,
                     (const uint8_t*)codes, k, n, (uint32_t*)packed);
  hipLaunchKernelGGL(k_pack_sm, dim3(grid_for((int64_t)k * (n / 64), 256)), dim3(256), 0, st,
                     (const uint32_t*)sm, k, n, (uint16_t*)scale, (uint16_t*)minv);
}

void launch_pack_f16(const void* w, int32_t k, int32_t n, void* wt, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_f16, dim3((unsigned)(n / 64), (unsigned)(k / 64)), dim3(256), 0, st,
                     (const uint16_t*)w, k, n, (uint16_t*)wt);
}

}  // namespace hp
