// Device-side work lists of one step, derived from the batch descriptor's device arrays.
//
// Each sequence is either a decode (one new token) or a prompt chunk (several new tokens at
// offset num_cached), the two kinds a chunked-prefill iteration mixes ("Chunked prefill
// (stall-free batching), explained", "How it works, step by step"). One 1024-thread workgroup
// classifies the sequences and scans their work counts:
//   decode unit  = (sequence, first page, decode index) covering `split_pages` KV pages;
//   decode entry = (sequence, first unit, unit count) for the split merge;
//   prefill tile = (sequence, first query row) covering `q_tile` query rows, emitted last tile
//                  first so the tiles with the longest key range are dispatched first.
// The host computes the same counts from its mirrors to size the grids, so nothing is read back.
#include "common.h"

namespace {

constexpr int kThreads = 1024;

__device__ int block_exclusive_scan(int v, int* buf, int* total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int add = (t >= off) ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const int incl = buf[t];
  *total = buf[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* __restrict__ q_start,
                                                        const int32_t* __restrict__ num_cached,
                                                        int num_seqs, int split_pages, int q_tile,
                                                        int32_t* __restrict__ dec_units,
                                                        int32_t* __restrict__ dec_seqs,
                                                        int32_t* __restrict__ pre_tiles,
                                                        int32_t* __restrict__ counters) {
  __shared__ int buf[kThreads];
  if (threadIdx.x < hl::kPlanCounters) counters[threadIdx.x * hl::kCounterStride] = 0;
  int base_u = 0, base_d = 0, base_t = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += kThreads) {
    const int s = s0 + threadIdx.x;
    int units = 0, is_dec = 0, tiles = 0;
    if (s < num_seqs) {
      const int qlen = q_start[s + 1] - q_start[s];
      const int kv = num_cached[s] + qlen;
      if (qlen == 1) {
        const int pages = (kv + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
        units = (pages + split_pages - 1) / split_pages;
        is_dec = 1;
      } else if (qlen > 1) {
        tiles = (qlen + q_tile - 1) / q_tile;
      }
    }
    int tot_u, tot_d, tot_t;
    const int off_u = base_u + block_exclusive_scan(units, buf, &tot_u);
    const int off_d = base_d + block_exclusive_scan(is_dec, buf, &tot_d);
    const int off_t = base_t + block_exclusive_scan(tiles, buf, &tot_t);
    if (is_dec) {
      for (int u = 0; u < units; ++u) {
        dec_units[3 * (off_u + u)] = s;
        dec_units[3 * (off_u + u) + 1] = u * split_pages;
        dec_units[3 * (off_u + u) + 2] = off_d;
      }
      dec_seqs[3 * off_d] = s;
      dec_seqs[3 * off_d + 1] = off_u;
      dec_seqs[3 * off_d + 2] = units;
    }
    for (int t = 0; t < tiles; ++t) {
      pre_tiles[2 * (off_t + t)] = s;
      pre_tiles[2 * (off_t + t) + 1] = (tiles - 1 - t) * q_tile;
    }
    base_u += tot_u;
    base_d += tot_d;
    base_t += tot_t;
  }
}

}  // namespace

namespace hl {
hipError_t launch_plan(const int32_t* q_start, const int32_t* num_cached, int32_t num_seqs,
                       int32_t split_pages, int32_t q_tile, const Plan& plan, hipStream_t st) {
  if (num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, st, q_start, num_cached, num_seqs,
                     split_pages, q_tile, plan.dec_units, plan.dec_seqs, plan.pre_tiles,
                     plan.counters);
  return hipGetLastError();
}
}  // namespace hl
