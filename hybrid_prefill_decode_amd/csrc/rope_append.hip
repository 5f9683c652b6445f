// Rotary embedding of q and k and append of the new K/V rows into the paged cache.
//
// Prompt chunks and decodes alike write the keys and values of their new tokens into the KV
// cache before attending ("Chunked prefill (stall-free batching), explained", "How it works, step
// by step"); the cache is paged and addressed through a block table, token p of sequence s living
// in block table[s][p / 16] at slot p % 16. Pages keep one KV head contiguous (the head-before-
// token layout of "Gescheiden Prefill en Decode", section on sharded KV cache transfers): K pages
// are [16 tokens][d], V pages [d][16 tokens].
//
// RoPE (rotate-half): pair (j, j + d/2) of a q or k head turns by p * theta^(-2j/d). The d/2
// angles of a token are formed in fp64 (p up to 10^5 keeps full precision), their sine and cosine
// shared by all heads through LDS; the rotation itself is fp32. One workgroup per token; the
// kernel is HBM-bound (reads (Hq + 2 Hkv) d bf16 and writes as many).
#include "common.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void rope_append_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ num_cached, int num_seqs,
    const hl_bf16* __restrict__ qkv, hl_bf16* __restrict__ q_rot, hl_bf16* __restrict__ kpool,
    hl_bf16* __restrict__ vpool, long long num_blocks, const int32_t* __restrict__ table,
    int max_blocks, int Hq, int Hkv, int D, float theta) {
  __shared__ float cs[2][128];
  const int t = blockIdx.x;
  // sequence owning token row t: the last s with q_start[s] <= t
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int p = num_cached[s] + (t - q_start[s]);
  const int half = D >> 1;
  if (threadIdx.x < half) {
    const double omega = pow((double)theta, -2.0 * (double)threadIdx.x / (double)D);
    double sn, cn;
    sincos((double)p * omega, &sn, &cn);
    cs[0][threadIdx.x] = (float)cn;
    cs[1][threadIdx.x] = (float)sn;
  }
  __syncthreads();

  const int ld = (Hq + 2 * Hkv) * D;
  const hl_bf16* src = qkv + (size_t)t * ld;
  const int blk = table[(size_t)s * max_blocks + p / HL_BLOCK_SIZE];
  const bool blk_ok = blk >= 0 && (long long)blk < num_blocks;
  const int slot = p % HL_BLOCK_SIZE;

  // rotate the Hq query heads and the Hkv key heads (pairs (j, j + d/2))
  const int n_pairs = (Hq + Hkv) * half;
  for (int e = threadIdx.x; e < n_pairs; e += kThreads) {
    const int h = e / half, j = e - h * half;
    const float a = bf2f(src[h * D + j]), b = bf2f(src[h * D + j + half]);
    const float c = cs[0][j], sn = cs[1][j];
    const uint32_t ra = f2bf(a * c - b * sn), rb = f2bf(b * c + a * sn);
    if (h < Hq) {
      q_rot[(size_t)t * Hq * D + h * D + j] = (hl_bf16)ra;
      q_rot[(size_t)t * Hq * D + h * D + j + half] = (hl_bf16)rb;
    } else if (blk_ok) {
      const int kh = h - Hq;
      hl_bf16* page = kpool + ((size_t)blk * Hkv + kh) * HL_BLOCK_SIZE * D;
      page[kpage_off(slot, j / 8) + j % 8] = (hl_bf16)ra;
      page[kpage_off(slot, (j + half) / 8) + (j + half) % 8] = (hl_bf16)rb;
    }
  }
  // values: copied unrotated into the dim-major V page
  if (blk_ok) {
    const hl_bf16* vs = src + (Hq + Hkv) * D;
    for (int e = threadIdx.x; e < Hkv * D; e += kThreads) {
      const int kh = e / D, dd = e - kh * D;
      vpool[(((size_t)blk * Hkv + kh) * D + dd) * HL_BLOCK_SIZE + slot] = vs[e];
    }
  }
}

}  // namespace

namespace hl {
hipError_t launch_rope_append(const hl_layer_cfg& cfg, int32_t num_seqs, int32_t num_tokens,
                              const int32_t* q_start, const int32_t* num_cached,
                              const hl_bf16* qkv, hl_bf16* q_rot, hl_bf16* kpool,
                              hl_bf16* vpool, int64_t num_blocks, const int32_t* table,
                              int32_t max_blocks, hipStream_t st) {
  if (num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_append_kernel, dim3(num_tokens), dim3(kThreads), 0, st, q_start,
                     num_cached, num_seqs, qkv, q_rot, kpool, vpool, (long long)num_blocks, table,
                     max_blocks, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rope_theta);
  return hipGetLastError();
}
}  // namespace hl
