// Measurement probes, not part of the layer: what this GPU attains on the two
// resources the kernels are bound by, as the reference for their fractions.
//  * k_peak_read streams a buffer once with 16-byte non-temporal loads, four
//    per lane in flight, grid-stride over the given number of 256-thread
//    workgroups (the rate depends on it: at 2 per CU it reads 7.05 TB/s, at
//    8 per CU 6.0-6.1, measured; fewer streams keep HBM rows open longer).
//  * k_peak_mfma keeps 16 independent v_mfma_f32_16x16x32_f16 chains per wave
//    on 8 waves per CU (two per SIMD), operands in registers.
// Both fold what they read or computed into a value that decides a store, so
// no load or product can be dropped.
#include "common.h"

namespace hp {

namespace {

__global__ __launch_bounds__(256) void k_peak_read(const u32x4* __restrict__ x, uint64_t n16,
                                                   uint32_t* __restrict__ sink) {
  constexpr int U = 4;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(x + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(512) void k_peak_mfma(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(1e-3f * (float)((lane + e) & 15));
    b[e] = (_Float16)(1e-3f * (float)((lane * 3 + e) & 15));
  }
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == -1.0f) sink[blockIdx.x * 8 + (threadIdx.x >> 6)] = __builtin_bit_cast(uint32_t, s);
}

}  // namespace

}  // namespace hp

using namespace hp;

extern "C" {

hp_status hp_peak_read(const void* x, uint64_t bytes, int32_t workgroups, uint32_t* sink,
                       void* stream) {
  if (!x || !sink) return fail(HP_ERR_NULL, "NULL pointer");
  if (((uintptr_t)x & 15) || (bytes & 15)) return fail(HP_ERR_SHAPE, "x and bytes: multiples of 16");
  if (workgroups < 1) return fail(HP_ERR_SHAPE, "workgroups < 1");
  hipLaunchKernelGGL(k_peak_read, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)x, bytes / 16, sink);
  return launch_ok("k_peak_read");
}

hp_status hp_peak_mfma(int32_t iters, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!sink) return fail(HP_ERR_NULL, "NULL pointer");
  if (iters < 1 || workgroups < 1) return fail(HP_ERR_SHAPE, "iters and workgroups must be >= 1");
  hipLaunchKernelGGL(k_peak_mfma, dim3((unsigned)workgroups), dim3(512), 0, (hipStream_t)stream,
                     iters, sink);
  return launch_ok("k_peak_mfma");
}

}  // extern "C"
