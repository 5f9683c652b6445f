// Per-token preparation pass in front of a normed linear layer.
//
// RMSNorm(x) * g W^T is computed as r * ((x * g) W^T) with r = 1 / sqrt(mean(x^2) + eps): the
// row scale r commutes with the product, so the GEMM consumes bf16(x * g) (exactly x when the
// gain is 1) and applies r to its fp32 accumulators. Rounding the normalised activation to bf16
// before the product is thereby avoided.
//
// The first pass of a step also records, per token row, the absolute position (num_cached + row
// offset within its sequence), the physical KV block of that position (block table lookup), and
// the rotary cos/sin of every pair j < d/2 at that position (angles formed in fp64), which the
// QKV GEMM epilogue uses to rotate q and k and to append K/V ("Chunked prefill (stall-free
// batching), explained", "How it works, step by step": new tokens write their K/V into the cache).
// When asked, kPlanWorkgroups extra workgroups of that pass build the step's attention work lists
// (plan_core.h), which saves the step a separate launch.
#include "plan_core.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxVec = 8;

template <bool TOKEN_INFO>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const hl_bf16* __restrict__ x, const hl_bf16* __restrict__ gain, hl_bf16* __restrict__ xg,
    float* __restrict__ rscale, int cols, float eps, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ num_cached, int num_seqs, const int32_t* __restrict__ table,
    int max_blocks, long long num_blocks, int D, float theta, int32_t* __restrict__ tok_pos,
    int32_t* __restrict__ tok_blk, float2* __restrict__ rope_cs, hl::Plan plan, int rows) {
  // with the work lists asked for, the first workgroups build them (dispatched first: their
  // chain of loads and scans is the longest of the launch) and the rows follow
  const int nlists = TOKEN_INFO ? (int)gridDim.x - rows : 0;
  if ((int)blockIdx.x < nlists) {
    __shared__ hl::plan::Shared<kThreads> sh;
    hl::plan::build<kThreads>(q_start, num_cached, num_seqs, table, max_blocks, plan, sh,
                              blockIdx.x, nlists);
    return;
  }
  const int row = blockIdx.x - nlists;
  if (TOKEN_INFO) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (q_start[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int p = num_cached[lo] + (row - q_start[lo]);
    const int half = D >> 1;
    if (threadIdx.x == 0) {
      const int blk = table[(size_t)lo * max_blocks + p / HL_BLOCK_SIZE];
      const bool decode = q_start[lo + 1] - q_start[lo] == 1;
      tok_pos[row] = p | (decode ? hl::kDecodeBit : 0);
      tok_blk[row] = (blk >= 0 && (long long)blk < num_blocks) ? blk : -1;
    }
    for (int j = threadIdx.x; j < half; j += kThreads) {
      const double omega = pow((double)theta, -2.0 * (double)j / (double)D);
      double sn, cn;
      sincos((double)p * omega, &sn, &cn);
      rope_cs[(size_t)row * half + j] = make_float2((float)cn, (float)sn);
    }
  }
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)row * cols);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gain);
  u32x4* yr = reinterpret_cast<u32x4*>(xg + (size_t)row * cols);
  const int nvec = cols / 8;
  u32x4 held[kMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int v = threadIdx.x + i * kThreads;
    if (v < nvec) {
      const u32x4 p = xr[v];
      held[i] = p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf_lo(p[e]), b = bf_hi(p[e]);
        ss += a * a + b * b;
      }
    }
  }
  for (int v = threadIdx.x + kMaxVec * kThreads; v < nvec; v += kThreads) {
    const u32x4 p = xr[v];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf_lo(p[e]), b = bf_hi(p[e]);
      ss += a * a + b * b;
    }
  }
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  __shared__ float part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
    rscale[row] = rsqrtf(tot / (float)cols + eps);
  }
  auto emit = [&](int v, u32x4 p) {
    const u32x4 g = gr[v];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf2(bf_lo(p[e]) * bf_lo(g[e]), bf_hi(p[e]) * bf_hi(g[e]));
    yr[v] = o;
  };
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int v = threadIdx.x + i * kThreads;
    if (v < nvec) emit(v, held[i]);
  }
  for (int v = threadIdx.x + kMaxVec * kThreads; v < nvec; v += kThreads) emit(v, xr[v]);
}

}  // namespace

namespace hl {

hipError_t launch_prep(const hl_bf16* x, const hl_bf16* gain, hl_bf16* xg, float* rscale,
                       int32_t rows, int32_t cols, float eps, const TokenInfo* ti,
                       hipStream_t st, const Plan* plan) {
  if (rows <= 0) return hipSuccess;
  if (ti) {
    const Plan pl = plan ? *plan : Plan{};
    hipLaunchKernelGGL(prep_kernel<true>, dim3(rows + (plan ? hl::kPlanWorkgroups : 0)),
                       dim3(kThreads), 0, st, x,
                       gain, xg, rscale, cols, eps, ti->q_start, ti->num_cached, ti->num_seqs,
                       ti->table, ti->max_blocks, (long long)ti->num_blocks, ti->head_dim,
                       ti->rope_theta, ti->tok_pos, ti->tok_blk, ti->rope_cs, pl, rows);
  } else {
    hipLaunchKernelGGL(prep_kernel<false>, dim3(rows), dim3(kThreads), 0, st, x, gain, xg, rscale,
                       cols, eps, nullptr, nullptr, 0, nullptr, 0, 0LL, 0, 0.f, nullptr, nullptr,
                       nullptr, Plan{}, rows);
  }
  return hipGetLastError();
}

}  // namespace hl
