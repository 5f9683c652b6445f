// Token-batched linear layer for batches of few tokens (decode-heavy iterations).
//
// With a handful of token rows, a linear layer is a stream of its weight matrix: each weight is
// used by as many multiply-adds as there are tokens, far below the matrix cores' ratio of work to
// HBM bytes, so the time is the weight bytes over HBM bandwidth (decode-heavy batches are bound by
// reads of weights and KV: chunked-prefill page, "Simulated numbers: choosing the budget"; chapter
// 7.8, "The Roofline Picture"). One tile per workgroup would leave most compute units idle (a
// 6144-column projection is 48 tiles of 128 columns), so this path splits K as well: workgroup
// (n-tile, k-chunk) computes the 64 output columns of its tile over its K range for all M (<= 64)
// rows, writing fp32 partials [chunk][M][N]; an epilogue kernel sums the chunks in a fixed order
// (deterministic) and applies the layer's epilogue (plain, residual, SwiGLU, or RoPE + KV append).
//
// Each wave owns 16 columns: per 32-deep k-step it loads one 16-byte W fragment per lane (16 rows
// x 64 bytes) and the matching A fragments (A is small and stays in L2), and issues one
// 16 x 16 x 32 MFMA per 16-row block of A. Four k-steps of fragments are prefetched ahead of the
// MFMAs that use them, so each wave keeps 4 KB of weights in flight.
#include <algorithm>

#include "gemm_core.h"

namespace {

constexpr int kCols = 64, kU = 4;  // (kThreads = 256 from gemm_core.h)

// partial[kc][m][n] (m < M) of the workgroup's 64 NW columns, k-steps [s0, s1) of 32. Wave w
// owns NW column blocks of 16; each A fragment feeds NW MFMAs and each W fragment MB, so with
// NW = MB the wave loads as many A bytes (from L2) as W bytes (from HBM).
template <int MB, int NW>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const hl_bf16* __restrict__ A,
                                                          const hl_bf16* __restrict__ W,
                                                          float* __restrict__ part, int M, int N,
                                                          int K, int steps_per_chunk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kCols * NW + 16 * NW * wave;
  const int kc = blockIdx.y;
  const int nks = K / 32;
  const int s0 = kc * steps_per_chunk, s1 = min(nks, s0 + steps_per_chunk);
  const int kq = lane >> 4;
  const hl_bf16* wp = W + (size_t)(n0 + (lane & 15)) * K + 8 * kq;
  const hl_bf16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ap[mb] = A + (size_t)min(16 * mb + (lane & 15), M - 1) * K + 8 * kq;
  f32x4 acc[MB][NW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[mb][t] = f32x4{};
  u32x4 wf[kU][NW], af[kU][MB];
  auto load = [&](int s, int u) {
    const int ss = min(s, s1 - 1);  // past the end: re-read the last step (unused)
#pragma unroll
    for (int t = 0; t < NW; ++t)
      wf[u][t] = *reinterpret_cast<const u32x4*>(wp + (size_t)16 * t * K + 32 * ss);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) af[u][mb] = *reinterpret_cast<const u32x4*>(ap[mb] + 32 * ss);
  };
#pragma unroll
  for (int u = 0; u < kU; ++u) load(s0 + u, u);
  for (int s = s0; s < s1; s += kU) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s + u < s1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int t = 0; t < NW; ++t) acc[mb][t] = mfma16x16x32(af[u][mb], wf[u][t], acc[mb][t]);
      }
      load(s + kU + u, u);  // refill this slot with the step kU ahead
    }
  }
  float* pp = part + ((size_t)kc * M) * N + n0 + (lane & 15);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mb + 4 * kq + r;
      if (m < M) {
#pragma unroll
        for (int t = 0; t < NW; ++t) pp[(size_t)m * N + 16 * t] = acc[mb][t][r];
      }
    }
}

// sum of the chunks of elements (m, n) and (m, n + 1), in chunk order
HL_DEV f32x2 chunk_sum2(const float* __restrict__ part, int chunks, int M, int N, int m, int n) {
  const size_t stride = (size_t)M * N;
  const float* p = part + (size_t)m * N + n;
  f32x2 v = {0.f, 0.f};
  int kc = 0;
  for (; kc + 4 <= chunks; kc += 4) {
    f32x2 t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = *reinterpret_cast<const f32x2*>(p + (kc + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) v += t[u];
  }
  for (; kc < chunks; ++kc) v += *reinterpret_cast<const f32x2*>(p + kc * stride);
  return v;
}

// plain / residual / SwiGLU epilogue over the summed partials; one thread per pair of
// consecutive output columns
__global__ __launch_bounds__(kThreads) void skinny_epilogue(const float* __restrict__ part,
                                                            int chunks, int M, int N,
                                                            hl_bf16* __restrict__ C, hl::GemmEpi ep) {
  const int out_n = ep.kind == HL_EPI_SWIGLU ? N / 2 : N;
  const long i = (long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long)M * (out_n / 2)) return;
  const int m = (int)(i / (out_n / 2)), j = 2 * (int)(i % (out_n / 2));
  const float rs = ep.row_scale ? ep.row_scale[m] : 1.f;
  f32x2 v;
  if (ep.kind == HL_EPI_SWIGLU) {
    const f32x2 g = chunk_sum2(part, chunks, M, N, m, j) * rs;
    const f32x2 u = chunk_sum2(part, chunks, M, N, m, N / 2 + j) * rs;
    v = f32x2{g[0] / (1.f + __expf(-g[0])) * u[0], g[1] / (1.f + __expf(-g[1])) * u[1]};
  } else {
    v = chunk_sum2(part, chunks, M, N, m, j) * rs;
  }
  const size_t o = (size_t)m * out_n + j;
  if (ep.kind == HL_EPI_RESIDUAL) {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(ep.residual + o);
    v[0] += bf_lo(r);
    v[1] += bf_hi(r);
  }
  *reinterpret_cast<uint32_t*>(C + o) = pack_bf2(v[0], v[1]);
}

// RoPE + KV-append epilogue: workgroup (row m, 256 columns = 256 / HD heads); every thread sums
// two columns into LDS, then thread (head, chunk c) rotates the 8 pairs (8c + e, HD/2 + 8c + e)
template <int HD>
__global__ __launch_bounds__(kThreads) void skinny_rope_epilogue(const float* __restrict__ part,
                                                                 int chunks, int M, int N,
                                                                 hl::GemmEpi ep) {
  __shared__ float row[2 * kThreads];
  const int m = blockIdx.y, c0 = blockIdx.x * 2 * kThreads;
  const float rs = ep.row_scale ? ep.row_scale[m] : 1.f;
  const int col = c0 + 2 * threadIdx.x;
  if (col < N) {
    const f32x2 v = chunk_sum2(part, chunks, M, N, m, col) * rs;
    row[2 * threadIdx.x] = v[0];
    row[2 * threadIdx.x + 1] = v[1];
  }
  __syncthreads();
  constexpr int kChunks = HD / 16, kHeads = 2 * kThreads / HD;
  if (threadIdx.x >= kHeads * kChunks) return;
  const int hl_ = threadIdx.x / kChunks, c = threadIdx.x % kChunks;
  const int gh = c0 / HD + hl_;
  if (gh * HD >= N) return;
  float a[8], b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = row[hl_ * HD + 8 * c + e];
    b[e] = row[hl_ * HD + HD / 2 + 8 * c + e];
  }
  const int pos = ep.tok_pos[m];
  rope_store_vals<HD>(ep, m, gh, ep.tok_blk[m], pos & (HL_BLOCK_SIZE - 1),
                      (pos & hl::kDecodeBit) != 0, a, b, c);
}

}  // namespace

namespace hl {

// Shape of the launch, from a sweep of (nw, chunks) on the layer shapes at 16, 32 and 64 rows:
// column blocks per wave nw = the 16-row blocks of A (up to 4, as N allows), so A and W bytes per
// MFMA balance; chunks of K = enough for about 1024 waves (each owns 16 nw columns of one chunk)
// and for at most 64 k-steps per chunk, but no more than keeps the fp32 partials (written and read
// back, 8 M bytes per column and chunk) within half the weight bytes (2 K per column), and at
// least 4 k-steps each. Within 15 % of the sweep's best on every shape measured.
struct SkinnyShape {
  int nw, chunks, steps_per_chunk;
};
SkinnyShape skinny_shape(int m, int n, int k) {
  const int nks = k / 32;
  const int mb = std::min(4, (m + 15) / 16);
  int nw = 1;
  if (mb == 4 && n % (kCols * 4) == 0) nw = 4;
  else if (mb >= 2 && n % (kCols * 2) == 0) nw = 2;
  const int per = n / (16 * nw);
  int kcs = std::max((1024 + per - 1) / per, (nks + 63) / 64);
  kcs = std::min(kcs, std::max(1, k / (8 * std::max(m, 1))));
  kcs = std::max(1, std::min(kcs, nks / 4));
  SkinnyShape sh;
  sh.nw = nw;
  sh.steps_per_chunk = (nks + kcs - 1) / kcs;
  sh.chunks = (nks + sh.steps_per_chunk - 1) / sh.steps_per_chunk;
  return sh;
}

size_t skinny_workspace_bytes(int m, int n, int k) {
  return (size_t)skinny_shape(m, n, k).chunks * m * n * 4;
}

hipError_t launch_gemm_skinny(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                              const GemmEpi& epi, float* part, hipStream_t st) {
  const SkinnyShape sh = skinny_shape(m, n, k);
  const int chunks = sh.chunks, spc = sh.steps_per_chunk, nw = sh.nw;
  const dim3 grid(n / (kCols * nw), chunks);
  const int mb = (m + 15) / 16;
#define HL_SKINNY(MB_, NW_)                                                                  \
  hipLaunchKernelGGL((skinny_kernel<MB_, NW_>), grid, dim3(kThreads), 0, st, a, w, part, m, n, \
                     k, spc)
  if (mb == 1) HL_SKINNY(1, 1);
  else if (mb == 2) { if (nw == 2) HL_SKINNY(2, 2); else HL_SKINNY(2, 1); }
  else if (mb == 3) { if (nw == 2) HL_SKINNY(3, 2); else HL_SKINNY(3, 1); }
  else if (nw == 4) HL_SKINNY(4, 4);
  else if (nw == 2) HL_SKINNY(4, 2);
  else HL_SKINNY(4, 1);
#undef HL_SKINNY
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (epi.kind == kEpiRopeAppend) {
    const dim3 eg((unsigned)((n + 2 * kThreads - 1) / (2 * kThreads)), (unsigned)m);
    if (epi.head_dim == 128)
      hipLaunchKernelGGL(skinny_rope_epilogue<128>, eg, dim3(kThreads), 0, st, part, chunks, m, n, epi);
    else
      hipLaunchKernelGGL(skinny_rope_epilogue<64>, eg, dim3(kThreads), 0, st, part, chunks, m, n, epi);
  } else {
    const int out_n = epi.kind == HL_EPI_SWIGLU ? n / 2 : n;
    const long items = (long)m * (out_n / 2);
    hipLaunchKernelGGL(skinny_epilogue, dim3((unsigned)((items + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, part, chunks, m, n, c, epi);
  }
  return hipGetLastError();
}

}  // namespace hl
