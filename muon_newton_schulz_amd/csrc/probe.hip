// MFMA-only ceiling probe (measurement aid, built as libmns_probe.so; not on the optimizer
// path). Every compute unit runs 8 workgroups of 4 waves; each wave issues back-to-back
// v_mfma_f32_32x32x16_f16 on 4 independent accumulators, its operands rotating through 8
// register fragments, with no memory access inside the loop. The launch's rate is therefore
// bounded only by the matrix pipes and by the clock the part holds under that load.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "mns_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBlocksPerCU = 8;
constexpr int kMaxBlocks = 512 * kBlocksPerCU;   // room for up to 512 compute units
constexpr int kMfmaPerIter = 8;

// Per-thread results (keeps the accumulators live); written with ordinary vector stores.
__device__ float g_sink[kMaxBlocks * kThreads];

// 8 float16 values in [-1, 1] (steps of 1/1000) from a linear congruential sequence.
__device__ __forceinline__ half8 fragment(unsigned s, bool zero) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s = s * 1664525u + 1013904223u;
    const int q = (int)((s >> 16) % 2001u) - 1000;
    h[i] = zero ? (_Float16)0.f : (_Float16)((float)q * 1e-3f);
  }
  return h;
}

__global__ __launch_bounds__(kThreads) void k_mfma_only(int iters, int zero) {
  const unsigned t = blockIdx.x * kThreads + threadIdx.x;
  half8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = fragment(t * 16u + i, zero != 0);
    b[i] = fragment(t * 16u + 8u + i, zero != 0);
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[j], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j + 1], b[j + 1], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j + 2], b[j + 2], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j + 3], b[j + 3], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  g_sink[t] = s;
}

int g_blocks = 0;   // blocks of the last launch (bounds the checksum read)

}  // namespace

extern "C" int mns_probe_mfma_launch(int iters, int zero_operands, void* stream,
                                     double* flops_per_launch) {
  if (iters < 1 || iters > 1000000 || !flops_per_launch) return 4;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 6;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 6;
  int blocks = cus * kBlocksPerCU;
  if (blocks < 1) return 6;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(k_mfma_only, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, iters,
                     zero_operands ? 1 : 0);
  if (hipGetLastError() != hipSuccess) return 6;
  g_blocks = blocks;
  *flops_per_launch =
      (double)blocks * (kThreads / 64) * iters * kMfmaPerIter * (2.0 * 32 * 32 * 16);
  return 0;
}

extern "C" int mns_probe_mfma_checksum(int n, double* sum) {
  if (n < 1 || n > 65536 || !sum || g_blocks == 0 || n > g_blocks * kThreads) return 4;
  std::vector<float> h(n);
  if (hipDeviceSynchronize() != hipSuccess) return 6;
  if (hipMemcpyFromSymbol(h.data(), HIP_SYMBOL(g_sink), n * sizeof(float), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return 6;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += std::fabs((double)h[i]);
  *sum = s;
  return 0;
}
