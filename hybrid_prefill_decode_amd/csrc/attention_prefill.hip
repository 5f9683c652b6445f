// Ragged causal attention of prompt chunks over their paged prefix plus themselves.
//
// A chunk of n new tokens at offset c attends to c + n keys: the cached prefix and, causally,
// the chunk itself; query position p sees keys 0..p ("Chunked prefill (stall-free batching),
// explained", "How it works, step by step"; "7.8 Disaggregated Prefill/Decode & Chunked Prefill",
// "Attention on Partial KV Caches"). Query head h reads KV head h / (Hq / Hkv) (the same chapter's
// GQA exercise). The new K/V rows are already in the pages when this kernel runs, so prefix and
// chunk keys are read the same way, through the block table.
//
// Work: one 256-thread workgroup per (128-row query tile, query head); wave w owns query rows
// 32w..32w+31. Keys advance 64 at a time (four 16-token pages) through a double-buffered LDS
// stage shared by the 4 waves. Scores are formed transposed, S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16, so each lane holds the keys of ONE query and the online-softmax max
// needs a single cross-lane exchange; P^T then feeds O^T = V^T P^T straight from registers (the
// k-slot order of the second product follows the register order of the first). V pages are
// dim-major ([d][16 tokens]) so the V^T operand is read without a transpose. Memory work is
// interleaved with the matrix cores (sched_group_barrier): K fragment reads between the score
// MFMAs, and during the P V^T MFMAs the LDS writes of the next key tile and the global loads of
// the one after it, so a load has a whole step to arrive. Workgroups of the query heads that share a
// KV head are dispatched to the same XCD (workgroups go to the 8 XCDs round-robin) so their K/V
// tiles hit in that XCD's L2. Softmax runs in fp32 in the exp2 domain. Keys past a query's
// position are masked by select and V rows past the sequence end are zeroed before they reach LDS,
// so unused cache slots never reach the result.
//
// Split key ranges. A tile's work grows with its key range, so a batch whose prefill is a few
// tiles over a long cached prefix (a short chunk late in a long prompt), or whose last causal
// tiles are much longer than its first, would keep a few compute units busy while the rest idle.
// The plan then splits such tiles into parts of at most `pre_split` key tiles; each part keeps
// its own online-softmax state and writes its unnormalised o with (m, l), and a merge pass
// combines the parts of each (tile, head): m* = max m_j, l* = sum l_j 2^(m_j - m*),
// o = sum o_j 2^(m_j - m*) / l* — the same split-softmax merge as split-KV decode.
#include "attn_prefill_core.h"

namespace {

using hl::prefill::PrefillArgs;

// Bijection from dispatch order to work order that keeps consecutive work items on one XCD.
HL_DEV int xcd_item(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// One workgroup per work item. Positions map to items through prefill_item_at, so each XCD runs
// whole (entry, KV head) units, longest key ranges first, and the XCDs get near-equal work.
template <int D>
__global__ __launch_bounds__(hl::prefill::kThreads, 2) void prefill_attn_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int item = hl::prefill_item_at(xcd_item(blockIdx.x, gridDim.x), gridDim.x / a.Hq, a.Hq,
                                       a.Hkv);
  const uint64_t t0 = a.trace ? (uint64_t)wall_clock64() : 0;
  hl::prefill::prefill_item<D>(a, item / a.Hq, item % a.Hq, smem);
  if (a.trace) {
    __syncthreads();
    hl::record_item(a.trace, item, t0);
  }
}

// Combine the parts of each split tile. One workgroup per (split tile, query head, block of
// kMergeRows query rows); each row is covered by kThreads / kMergeRows threads, each over a
// contiguous run of the head dimension, and the parts' loads are independent of one another.
constexpr int kMergeRows = 16;

template <int D>
__global__ __launch_bounds__(hl::prefill::kThreads) void prefill_merge_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ merges,
    const float* __restrict__ part_o, const float2* __restrict__ part_ml, int Hq,
    hl_bf16* __restrict__ attn_out) {
  constexpr int QT = hl::kPrefillQTile, TPR = hl::prefill::kThreads / kMergeRows, DPT = D / TPR;
  static_assert(DPT % 4 == 0, "whole 16-byte pieces per thread");
  const int e = blockIdx.x, h = blockIdx.y;
  const int s = merges[4 * e], r0 = merges[4 * e + 1], slot0 = merges[4 * e + 2],
            np = merges[4 * e + 3];
  const int row = blockIdx.z * kMergeRows + threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * DPT;
  const int qs = q_start[s];
  if (r0 + row >= q_start[s + 1] - qs) return;
  const size_t pstride = (size_t)Hq * QT;  // rows between consecutive slots
  const size_t prow = ((size_t)slot0 * Hq + h) * QT + row;
  float mx = -1e30f;
  for (int j = 0; j < np; ++j) mx = fmaxf(mx, part_ml[prow + j * pstride].x);
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
  float lsum = 0.f;
#pragma unroll 4
  for (int j = 0; j < np; ++j) {
    const float2 ml = part_ml[prow + j * pstride];
    const float wj = exp2f(ml.x - mx);
    lsum += ml.y * wj;
    const f32x4* src = reinterpret_cast<const f32x4*>(part_o + (prow + j * pstride) * D + d0);
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) {
      const f32x4 v = src[i];
      acc[4 * i] += v[0] * wj;
      acc[4 * i + 1] += v[1] * wj;
      acc[4 * i + 2] += v[2] * wj;
      acc[4 * i + 3] += v[3] * wj;
    }
  }
  const float inv = 1.f / lsum;
  hl_bf16* op = attn_out + ((size_t)(qs + r0 + row) * Hq + h) * D + d0;
#pragma unroll
  for (int i = 0; i < DPT / 4; ++i)
    *reinterpret_cast<u32x2*>(op + 4 * i) = u32x2{pack_bf2(acc[4 * i] * inv, acc[4 * i + 1] * inv),
                                                  pack_bf2(acc[4 * i + 2] * inv, acc[4 * i + 3] * inv)};
}

}  // namespace

namespace hl {

hipError_t launch_prefill_merge(const hl_layer_cfg& cfg, const int32_t* q_start, const Plan& plan,
                                hl_bf16* attn_out, hipStream_t st) {
  if (plan.n_pre_merge <= 0) return hipSuccess;
  const dim3 grid(plan.n_pre_merge, cfg.n_q_heads, kPrefillQTile / kMergeRows),
      block(prefill::kThreads);
  if (cfg.head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, block, 0, st, q_start, plan.pre_merge,
                       plan.pre_part_o, plan.pre_part_ml, cfg.n_q_heads, attn_out);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, block, 0, st, q_start, plan.pre_merge,
                       plan.pre_part_o, plan.pre_part_ml, cfg.n_q_heads, attn_out);
  return hipGetLastError();
}

using prefill::PrefillArgs;
using prefill::PrefillSmem;
using prefill::kThreads;

hipError_t launch_prefill_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                    const int32_t* num_cached, const hl_bf16* q_rot,
                                    const hl_bf16* kpool, const hl_bf16* vpool,
                                    int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                                    const Plan& plan, hl_bf16* attn_out, hipStream_t st) {
  if (plan.n_pre_tiles <= 0) return hipSuccess;
  const float scale = cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(plan.n_pre_tiles * cfg.n_q_heads), block(kThreads);
  const PrefillArgs args{q_start, num_cached, q_rot, kpool, vpool, (long long)num_blocks, table,
                         max_blocks, plan.pre_tiles, cfg.n_q_heads, cfg.n_kv_heads, scale_log2,
                         attn_out, plan.pre_part_o, plan.pre_part_ml, plan.trace};
  if (cfg.head_dim == 128) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_attn_kernel<128>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, PrefillSmem<128>::kTotal);
      (void)hipGetLastError();
      attr = true;
    }
    hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, block, PrefillSmem<128>::kTotal, st, args);
  } else {
    hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, block, PrefillSmem<64>::kTotal, st, args);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_prefill_merge(cfg, q_start, plan, attn_out, st);
}

}  // namespace hl
