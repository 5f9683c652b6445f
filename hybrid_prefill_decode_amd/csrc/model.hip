// Model-level pieces around the layer stack: token embedding, the last row of each sequence,
// and the greedy pick over the vocabulary.
//
// One iteration of chunked prefill runs every layer over the flattened hybrid batch, and a
// request whose last prompt chunk completes samples its first token from that same pass ("Chunked
// prefill (stall-free batching), explained", "How it works, step by step"); the logits are taken
// for the last position only and the greedy choice is their argmax (chapter 7.8, the prefill
// worker's listing). Decodes take their next token the same way. All three kernels are HBM-bound
// copies or scans.
#include "common.h"

namespace {

constexpr int kThreads = 256;

// x[t, :] = table[tokens[t], :], 16-byte chunks, grid-stride. Ids were checked on the host.
__global__ __launch_bounds__(kThreads) void embed_kernel(const int32_t* __restrict__ tokens,
                                                         const hl_bf16* __restrict__ table,
                                                         hl_bf16* __restrict__ x, int T, int H,
                                                         int vocab) {
  const int chunks = H / 8;
  const long total = (long)T * chunks;
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    const int t = (int)(i / chunks), c = (int)(i % chunks);
    const int id = min(max(tokens[t], 0), vocab - 1);
    *reinterpret_cast<u32x4*>(x + (size_t)t * H + 8 * c) =
        *reinterpret_cast<const u32x4*>(table + (size_t)id * H + 8 * c);
  }
}

// rows[s, :] = x[q_start[s + 1] - 1, :]: the last new token of each sequence
__global__ __launch_bounds__(kThreads) void last_rows_kernel(const int32_t* __restrict__ q_start,
                                                             const hl_bf16* __restrict__ x,
                                                             hl_bf16* __restrict__ rows, int S,
                                                             int H) {
  const int s = blockIdx.x;
  const int r = q_start[s + 1] - 1;
  for (int c = threadIdx.x; c < H / 8; c += kThreads)
    *reinterpret_cast<u32x4*>(rows + (size_t)s * H + 8 * c) =
        *reinterpret_cast<const u32x4*>(x + (size_t)r * H + 8 * c);
}

// (value, index) order of the greedy pick: NaN above everything (as a plain argmax scan would
// stop there), then the larger value, then the smaller index
HL_DEV bool better(float v1, int i1, float v2, int i2) {
  const bool n1 = v1 != v1, n2 = v2 != v2;
  if (n1 != n2) return n1;
  if (!n1 && v1 != v2) return v1 > v2;
  return i1 < i2;
}

// out[s] = first index of the largest of logits[s, 0 .. V-1] (bf16); one workgroup per row
__global__ __launch_bounds__(kThreads) void argmax_kernel(const hl_bf16* __restrict__ logits,
                                                          int V, int32_t* __restrict__ out) {
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const hl_bf16* row = logits + (size_t)blockIdx.x * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int base = 8 * threadIdx.x; base < V; base += 8 * kThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + base);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf_lo(v[e]), hi = bf_hi(v[e]);
      if (better(lo, base + 2 * e, bv, bi)) bv = lo, bi = base + 2 * e;
      if (better(hi, base + 2 * e + 1, bv, bi)) bv = hi, bi = base + 2 * e + 1;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (better(ov, oi, bv, bi)) bv = ov, bi = oi;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sv[wave] = bv, si[wave] = bi;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) bv = sv[w], bi = si[w];
    out[blockIdx.x] = bi;
  }
}

}  // namespace

namespace hl {

hipError_t launch_embed(const int32_t* tokens, const hl_bf16* table, hl_bf16* x, int T, int H,
                        int vocab, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const long chunks = (long)T * (H / 8);
  const int grid = (int)std::min<long>((chunks + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(embed_kernel, dim3(grid), dim3(kThreads), 0, st, tokens, table, x, T, H, vocab);
  return hipGetLastError();
}

hipError_t launch_last_rows(const int32_t* q_start, const hl_bf16* x, hl_bf16* rows, int S, int H,
                            hipStream_t st) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(last_rows_kernel, dim3(S), dim3(kThreads), 0, st, q_start, x, rows, S, H);
  return hipGetLastError();
}

hipError_t launch_argmax(const hl_bf16* logits, int S, int V, int32_t* out, hipStream_t st) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3(S), dim3(kThreads), 0, st, logits, V, out);
  return hipGetLastError();
}

}  // namespace hl
