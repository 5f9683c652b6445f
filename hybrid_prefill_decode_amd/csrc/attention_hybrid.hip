// Fused hybrid attention: the prefill work items and the decode work units of one hybrid batch run
// in a single launch, so the compute-bound prefill path and the bandwidth-bound decode path
// overlap on every compute unit. The two attention paths of a hybrid step are independent and use
// different resources (prefill the matrix cores, decode the HBM bandwidth), so running them side
// by side hides one behind the other ("ConfluxServe" summary, "Why can linear layers be batched
// but attention cannot?", which splits the GPU's compute units between the paths); a fused
// prefill-decode attention kernel is what turns that overlap into step time ("Chunked prefill
// (stall-free batching), explained", "Simulated numbers: choosing the budget").
//
// Persistent workers, two per compute unit. Workers 0..P-1 start on prefill items, the rest on
// decode units; workgroups are dealt to the compute units one each before any gets a second, so
// every unit holds one worker of each kind: the split of the units between the paths happens
// inside each unit, where the matrix cores and the memory pipeline are both kept busy. Work is
// claimed from device counters that the step's plan kernel zeroes: a prefill item comes from the
// queue of the worker's XCD (the query heads of one KV head are consecutive items, so their K/V
// tiles hit in that XCD's L2), then from the other XCDs' queues; a decode unit from the single
// decode queue. A worker that drains its own kind helps with the other; every worker exits once all
// queues are empty. Each item runs the same code as in the separate kernels, so the results are
// bit-identical to theirs.
#include "attn_decode_core.h"
#include "attn_prefill_core.h"

namespace {

using hl::decode::DecodeArgs;
using hl::decode::DecodeLds;
using hl::prefill::PrefillArgs;
using hl::prefill::PrefillSmem;

constexpr int kThreads = 256;
static_assert(kThreads == hl::decode::kThreads && kThreads == hl::prefill::kThreads, "workgroup");

// first prefill item of XCD x's queue when n items are dealt to 8 XCDs in contiguous runs
HL_DEV int queue_begin(int x, int n) {
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r);
}

template <int D>
constexpr int kHybridLds = PrefillSmem<D>::kTotal > (int)sizeof(DecodeLds<D>)
                               ? PrefillSmem<D>::kTotal
                               : (int)sizeof(DecodeLds<D>);

// counters[0..7]: prefill queue of each XCD; counters[8]: decode queue.
//
// Queue sequence of a worker: a prefill worker visits its XCD's prefill queue, the other seven,
// then the decode queue (stage 8); a decode worker visits the decode queue (stage 0), then the
// eight prefill queues from its own XCD on. A claim is one atomic increment of the current stage's
// counter by thread 0, broadcast through LDS; everything else about the queues is computed by all
// threads alike, so control flow stays uniform across the workgroup (the only one-thread branches
// are the atomic and the LDS write).
struct Queues {
  int32_t* counters;
  int n_pre, n_dec, xcd;
  bool pre_worker;
  HL_DEV bool is_dec(int stage) const { return pre_worker ? stage == 8 : stage == 0; }
  HL_DEV int32_t* counter(int stage) const {
    return is_dec(stage) ? &counters[8] : &counters[(xcd + (pre_worker ? stage : stage - 1)) & 7];
  }
  // [begin, end) of the stage's items in claim numbering (prefill items first, then decode)
  HL_DEV void range(int stage, int& beg, int& end) const {
    if (is_dec(stage)) {
      beg = n_pre;
      end = n_pre + n_dec;
    } else {
      const int x = (xcd + (pre_worker ? stage : stage - 1)) & 7;
      beg = queue_begin(x, n_pre);
      end = queue_begin(x + 1, n_pre);
    }
  }
  // the claimed item for ticket i of `stage`, or -1 if that queue is drained
  HL_DEV int resolve(int stage, int i) const {
    int beg, end;
    range(stage, beg, end);
    return beg + i < end ? beg + i : -1;
  }
};

// one ticket of `stage` for the whole workgroup (called by every thread)
HL_DEV int wg_ticket(const Queues& qs, int stage, int* s_tick) {
  if (threadIdx.x == 0) *s_tick = atomicAdd(qs.counter(stage), 1);
  __syncthreads();
  const int t = *s_tick;
  __syncthreads();  // s_tick may be rewritten by the next claim
  return t;
}

// waiting claim from `stage` on (every thread; stage uniform); advances stage past drained queues;
// -1 when all are drained
HL_DEV int wg_claim(const Queues& qs, int& stage, int* s_tick) {
  for (; stage < 9; ++stage) {
    int beg, end;
    qs.range(stage, beg, end);
    if (beg >= end) continue;
    const int c = qs.resolve(stage, wg_ticket(qs, stage, s_tick));
    if (c >= 0) return c;
  }
  return -1;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void hybrid_attn_kernel(
    PrefillArgs pa, DecodeArgs da, int32_t* __restrict__ counters, int n_pre_items,
    int n_dec_items, int n_pre_workers) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_tick;
  const Queues qs{counters, n_pre_items, n_dec_items, (int)(blockIdx.x & 7),
                  (int)blockIdx.x < n_pre_workers};
  int stage = 0;
  int cur = wg_claim(qs, stage, &s_tick);
  while (cur >= 0) {
    // Decode units are short: thread 0 takes the next decode ticket now and publishes it after
    // the unit. Prefill items are long and few, so their next claim waits for the item's end
    // (a ticket taken early would reserve an item that an idle worker could have run).
    const bool ahead = stage < 9 && qs.is_dec(stage);
    int t = 0;
    if (threadIdx.x == 0 && ahead) t = atomicAdd(qs.counter(stage), 1);
    if (cur < n_pre_items) {
      hl::prefill::prefill_item<D>(pa, cur / pa.Hq, cur % pa.Hq, smem);
    } else {
      const int u = cur - n_pre_items;
      hl::decode::decode_unit<D>(da, u / da.Hkv, u % da.Hkv,
                                 *reinterpret_cast<DecodeLds<D>*>(smem));
    }
    int next;
    if (ahead) {
      if (threadIdx.x == 0) s_tick = t;
      __syncthreads();  // also: the item's LDS reads are done before the next item writes
      next = qs.resolve(stage, s_tick);
      __syncthreads();
      if (next < 0) {
        ++stage;
        next = wg_claim(qs, stage, &s_tick);
      }
    } else {
      __syncthreads();  // the item's LDS reads are done before the next item writes
      next = wg_claim(qs, stage, &s_tick);
    }
    cur = next;
  }
}

template <int D>
hipError_t launch(const PrefillArgs& pa, const DecodeArgs& da, int32_t* counters, int n_pre_items,
                  int n_dec_items, int cus, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(hybrid_attn_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kHybridLds<D>);
    (void)hipGetLastError();
    attr = true;
  }
  const int total = n_pre_items + n_dec_items;
  const int n_pre_workers = n_pre_items > 0 ? std::min(cus, n_pre_items) : 0;
  const int workers = std::min(2 * cus, total);
  hipLaunchKernelGGL(hybrid_attn_kernel<D>, dim3(workers), dim3(kThreads), kHybridLds<D>, st, pa,
                     da, counters, n_pre_items, n_dec_items, std::min(n_pre_workers, workers));
  return hipGetLastError();
}

}  // namespace

namespace hl {

hipError_t launch_hybrid_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                   const int32_t* num_cached, const hl_bf16* q_rot,
                                   const hl_bf16* q_lo, const hl_bf16* kpool,
                                   const hl_bf16* vpool, int64_t num_blocks, const int32_t* table,
                                   int32_t max_blocks, const Plan& plan, int32_t cus,
                                   hl_bf16* attn_out, hipStream_t st) {
  const int n_pre_items = plan.n_pre_tiles * cfg.n_q_heads;
  const int n_dec_items = plan.n_dec_units * cfg.n_kv_heads;
  if (n_pre_items + n_dec_items <= 0) return hipSuccess;
  const float scale = cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  const float scale_log2 = scale * 1.4426950408889634f;
  const PrefillArgs pa{q_start, num_cached, q_rot, kpool, vpool, (long long)num_blocks, table,
                       max_blocks, plan.pre_tiles, cfg.n_q_heads, cfg.n_kv_heads, scale_log2,
                       attn_out};
  const decode::DecodeArgs da{q_start,        num_cached,     q_rot,          q_lo,
                              kpool,          vpool,          (long long)num_blocks, table,
                              max_blocks,     plan.dec_units, plan.dec_seqs,  plan.split_pages,
                              cfg.n_q_heads,  cfg.n_kv_heads, scale_log2,     plan.dec_part,
                              attn_out};
  hipError_t e = cfg.head_dim == 128
                     ? launch<128>(pa, da, plan.counters, n_pre_items, n_dec_items, cus, st)
                     : launch<64>(pa, da, plan.counters, n_pre_items, n_dec_items, cus, st);
  if (e != hipSuccess || n_dec_items == 0) return e;
  return launch_decode_merge(cfg, q_start, plan, attn_out, st);
}

}  // namespace hl
