// RMSNorm over the token rows of the hybrid batch: y = x / sqrt(mean(x^2) + eps) * gain.
// One 256-thread workgroup per row; fp32 arithmetic; 16-byte loads and stores. HBM-bound:
// it reads and writes every element once (4 bytes of traffic per element).
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxVec = 8;  // row held in registers when cols <= 256 * 8 * 8

__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const hl_bf16* __restrict__ x,
                                                           const hl_bf16* __restrict__ gain,
                                                           hl_bf16* __restrict__ y, int cols,
                                                           float eps) {
  const int row = blockIdx.x;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)row * cols);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gain);
  u32x4* yr = reinterpret_cast<u32x4*>(y + (size_t)row * cols);
  const int nvec = cols / 8;
  u32x4 held[kMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    int v = threadIdx.x + i * kThreads;
    if (v < nvec) {
      u32x4 p = xr[v];
      held[i] = p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = bf_lo(p[e]), b = bf_hi(p[e]);
        ss += a * a + b * b;
      }
    }
  }
  for (int v = threadIdx.x + kMaxVec * kThreads; v < nvec; v += kThreads) {
    u32x4 p = xr[v];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = bf_lo(p[e]), b = bf_hi(p[e]);
      ss += a * a + b * b;
    }
  }
  // workgroup reduction: wave butterfly, then across the 4 waves through LDS
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  __shared__ float part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
  const float r = rsqrtf(tot / (float)cols + eps);

  auto emit = [&](int v, u32x4 p) {
    u32x4 g = gr[v];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = bf_lo(p[e]) * r * bf_lo(g[e]);
      float b = bf_hi(p[e]) * r * bf_hi(g[e]);
      o[e] = pack_bf2(a, b);
    }
    yr[v] = o;
  };
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    int v = threadIdx.x + i * kThreads;
    if (v < nvec) emit(v, held[i]);
  }
  for (int v = threadIdx.x + kMaxVec * kThreads; v < nvec; v += kThreads) emit(v, xr[v]);
}

}  // namespace

namespace hl {
hipError_t launch_rmsnorm(const hl_bf16* x, const hl_bf16* g, hl_bf16* y, int32_t rows,
                          int32_t cols, float eps, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(kThreads), 0, st, x, g, y, cols, eps);
  return hipGetLastError();
}
}  // namespace hl
