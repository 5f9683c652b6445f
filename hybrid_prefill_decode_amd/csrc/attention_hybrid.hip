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
// inside each unit, where the matrix cores and the memory pipeline are both kept busy.
//
// Queues. The items of each kind are dealt to 8 queues in contiguous runs of positions, one per
// XCD; prefill positions map to items through prefill_item_at (whole (entry, KV head) units per
// XCD, longest first, so the XCDs get near-equal prefill work and share K/V tiles in L2). A
// worker's first item needs no claim: the l-th worker of a kind on XCD x takes the l-th item of
// that kind's queue x. Further items are claimed from per-queue device counters (zeroed by the
// step's plan kernel, each on its own 256-byte line) that number the claims past those first
// items: a worker drains its own queue, then the other XCDs' queues of its kind, then helps with
// the other kind (except prefill workers of a decode-heavy launch), and exits once every queue it
// may take from is empty. A queue is read before it is incremented,
// so drained queues cost no atomic. (One shared decode counter serialised every claim at one
// memory location: with a few hundred workers that cost tens of microseconds per launch.)
// Each item runs the same code as in the separate kernels (and the same merges follow), so the
// results are bit-identical to theirs.
#include <type_traits>

#include "attn_decode_core.h"
#include "attn_prefill_core.h"

namespace {

using hl::decode::Carry;
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

// Queues 0..7: prefill items of XCD 0..7; queues 8..15: decode units of XCD 0..7 (decode units
// are numbered after the prefill items). Everything about the queues is computed by all threads
// alike, so control flow stays uniform across the workgroup; a claim is a peek and an atomic
// increment by thread 0, broadcast through LDS (the only one-thread branch).
struct Queues {
  int32_t* counters;
  int n_pre, n_dec;  // items of each kind
  int wp, w;         // prefill workers are blocks [0, wp), decode workers [wp, w)
  int xcd;           // this worker's XCD (blocks go to the 8 XCDs round-robin)
  bool pre_worker;
  HL_DEV int begin(int q) const {
    return q < 8 ? queue_begin(q, n_pre) : n_pre + queue_begin(q - 8, n_dec);
  }
  HL_DEV int end(int q) const {
    return q < 8 ? queue_begin(q + 1, n_pre) : n_pre + queue_begin(q - 7, n_dec);
  }
  // first block of queue q's kind on its XCD, and how many blocks of that kind it holds
  HL_DEV int first_block(int q) const {
    const int lo = q < 8 ? 0 : wp;
    return lo + (((q & 7) - lo) % 8 + 8) % 8;
  }
  HL_DEV int workers_on(int q) const {
    const int hi = q < 8 ? wp : w, f = first_block(q);
    return f < hi ? (hi - f + 7) / 8 : 0;
  }
  // items of queue q taken without a claim (one per worker of its kind on its XCD)
  HL_DEV int statics(int q) const { return min(workers_on(q), end(q) - begin(q)); }
  HL_DEV int32_t* counter(int q) const { return counters + q * hl::kCounterStride; }
  // queue of stage s (0..15): the worker's own kind from its own XCD on, then the other kind
  HL_DEV int queue_at(int s) const {
    const int own = pre_worker ? 0 : 8;
    return s < 8 ? own + ((xcd + s) & 7) : (8 - own) + ((xcd + s - 8) & 7);
  }
  // this worker's first item (no claim), or -1
  HL_DEV int first_item(int block) const {
    const int q = (pre_worker ? 0 : 8) + xcd;
    const int l = (block - first_block(q)) / 8;
    return l < statics(q) ? begin(q) + l : -1;
  }
  // item of claim ticket t of queue q, or -1 if the queue is drained
  HL_DEV int resolve(int q, int t) const {
    const int i = begin(q) + statics(q) + t;
    return (t >= 0 && i < end(q)) ? i : -1;
  }
};

// a claim from queue q for the whole workgroup (called by every thread): -1 if it is drained
HL_DEV int wg_claim_queue(const Queues& qs, int q, int* s_tick) {
  if (qs.begin(q) + qs.statics(q) >= qs.end(q)) return -1;  // nothing beyond the first items
  if (threadIdx.x == 0) {
    const int seen = __hip_atomic_load(qs.counter(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_tick = (qs.begin(q) + qs.statics(q) + seen < qs.end(q)) ? atomicAdd(qs.counter(q), 1) : -1;
  }
  __syncthreads();
  // every lane reads the same value; readfirstlane tells the compiler so, which keeps the item
  // index, and the loops it bounds, in scalar registers
  const int t = __builtin_amdgcn_readfirstlane(*s_tick);
  __syncthreads();  // s_tick may be rewritten by the next claim
  return qs.resolve(q, t);
}

// waiting claim from stage `stage` on (every thread; stage uniform); advances stage past drained
// queues up to `stages`; -1 when all of those are drained
HL_DEV int wg_claim(const Queues& qs, int& stage, int stages, int* s_tick) {
  for (; stage < stages; ++stage) {
    const int c = wg_claim_queue(qs, qs.queue_at(stage), s_tick);
    if (c >= 0) return c;
  }
  return -1;
}

// PF: decode units prefetch the next unit of their worker (attn_decode_core.h). Worth it when
// decode units dominate the launch; it costs registers, which the prefill items then spill.
template <int D, bool PF>
__global__ __launch_bounds__(kThreads, 2) void hybrid_attn_kernel(
    PrefillArgs pa, DecodeArgs da, int32_t* __restrict__ counters, int n_pre_items,
    int n_dec_items, int n_pre_workers, uint64_t* __restrict__ trace) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_tick;
  const Queues qs{counters, n_pre_items, n_dec_items, n_pre_workers, (int)gridDim.x,
                  (int)(blockIdx.x & 7), (int)blockIdx.x < n_pre_workers};
  // In a decode-heavy launch (PF) the prefill workers stop when the prefill queues are drained
  // instead of joining the decode units: one decode worker per compute unit already keeps HBM
  // busy, and the joining workers' start-up, the shorter units and the thinner tail of fewer
  // concurrent streams measured ~1.5 % faster over the launch on the 70B-shaped batch. Decode
  // workers still help with prefill items once the decode queues are drained.
  const int stages = (PF && qs.pre_worker) ? 8 : 16;
  int stage = 0;
  int cur = qs.first_item(blockIdx.x);
  if (cur < 0) cur = wg_claim(qs, stage, stages, &s_tick);
  while (cur >= 0) {
    if (cur < n_pre_items) {
      // prefill items are long and few: the next claim waits for the item's end (a ticket taken
      // early would reserve an item that an idle worker could have run)
      const uint64_t t0 = trace ? (uint64_t)wall_clock64() : 0;
      const int item = hl::prefill_item_at(cur, n_pre_items / pa.Hq, pa.Hq, pa.Hkv);
      hl::prefill::prefill_item<D>(pa, item / pa.Hq, item % pa.Hq, smem);
      __syncthreads();  // the item's LDS reads are done before the next item writes
      if (trace) hl::record_item(trace, item, t0);
      cur = wg_claim(qs, stage, stages, &s_tick);
      continue;
    }
    // A run of decode units. Thread 0 claims the next unit as the current one starts. With PF it
    // publishes the claim in LDS right away, where each wave reads it near the end of its pages
    // to start the next unit's loads (decode_item); without, the claim is published after the
    // unit, so its atomic's latency hides behind the unit.
    DecodeLds<D>& L = *reinterpret_cast<DecodeLds<D>*>(smem);
    if (PF) {
      if (threadIdx.x == 0) L.tick = hl::decode::kTickPending;
      __syncthreads();
    }
    Carry<D> cy;
    cy.item = -1;
    cy.has_pair = false;
    while (cur >= n_pre_items) {
      const int q = qs.queue_at(stage);
      int t = -1;
      if (threadIdx.x == 0 && q >= 8) {
        t = atomicAdd(qs.counter(q), 1);
        if (PF) {
          const int nx = qs.resolve(q, t);
          __hip_atomic_store(&L.tick, nx >= n_pre_items ? nx - n_pre_items : -1,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      const uint64_t t0 = trace ? (uint64_t)wall_clock64() : 0;
      const int seq_item = hl::decode::decode_item<D, PF>(da, cur - n_pre_items, L, cy);
      if (!PF && threadIdx.x == 0) s_tick = t;
      __syncthreads();  // the unit's LDS reads are done and thread 0's claim is visible
      int next;
      if (PF) {
        const int nd = __builtin_amdgcn_readfirstlane(L.tick);
        next = nd >= 0 ? nd + n_pre_items : -1;
      } else {
        next = q >= 8 ? qs.resolve(q, __builtin_amdgcn_readfirstlane(s_tick)) : -1;
      }
      if (trace) hl::record_item(trace, n_pre_items + seq_item, t0);
      __syncthreads();  // every wave has read the claim before thread 0 overwrites it
      if (PF && threadIdx.x == 0) L.tick = hl::decode::kTickPending;
      if (next < 0) {
        ++stage;
        next = wg_claim(qs, stage, stages, &s_tick);
      }
      cur = next;
      if (cur < 0) break;
    }
  }
}

template <int D, bool PF>
hipError_t launch(const PrefillArgs& pa, const DecodeArgs& da, int32_t* counters, int n_pre_items,
                  int n_dec_items, int cus, uint64_t* trace, hipStream_t st) {
  constexpr int lds = kHybridLds<D>;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(hybrid_attn_kernel<D, PF>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipGetLastError();
    attr = true;
  }
  const int total = n_pre_items + n_dec_items;
  const int n_pre_workers = n_pre_items > 0 ? std::min(cus, n_pre_items) : 0;
  const int workers = std::min(2 * cus, total);
  hipLaunchKernelGGL((hybrid_attn_kernel<D, PF>), dim3(workers), dim3(kThreads), lds, st,
                     pa, da, counters, n_pre_items, n_dec_items,
                     std::min(n_pre_workers, workers), trace);
  return hipGetLastError();
}

DecodeArgs decode_args(const hl_layer_cfg& cfg, const int32_t* q_start,
                               const int32_t* num_cached, const hl_bf16* q_rot,
                               const hl_bf16* q_lo, const hl_bf16* kpool, const hl_bf16* vpool,
                               int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                               const hl::Plan& plan, float scale_log2, hl_bf16* attn_out) {
  return DecodeArgs{q_start,        num_cached,     q_rot,          q_lo,
                            kpool,          vpool,          (long long)num_blocks, table,
                            max_blocks,     plan.dec_units, plan.dec_seqs,  plan.split_pages,
                            cfg.n_q_heads,  cfg.n_kv_heads, scale_log2,     plan.dec_part,
                            attn_out,       plan.n_dec_units * cfg.n_kv_heads, plan.dec_lpt};
}

float scale_log2_of(const hl_layer_cfg& cfg) {
  const float scale =
      cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  return scale * 1.4426950408889634f;
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
  const float sl2 = scale_log2_of(cfg);
  const PrefillArgs pa{q_start, num_cached, q_rot, kpool, vpool, (long long)num_blocks, table,
                       max_blocks, plan.pre_tiles, cfg.n_q_heads, cfg.n_kv_heads, sl2,
                       attn_out, plan.pre_part_o, plan.pre_part_ml, nullptr};
  const DecodeArgs da = decode_args(cfg, q_start, num_cached, q_rot, q_lo, kpool, vpool,
                                            num_blocks, table, max_blocks, plan, sl2, attn_out);
  auto go = [&](auto d, auto pf) {
    return launch<decltype(d)::value, decltype(pf)::value>(pa, da, plan.counters, n_pre_items,
                                                           n_dec_items, cus, plan.trace, st);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  using On = std::true_type;
  using Off = std::false_type;
  hipError_t e = cfg.head_dim == 128 ? (plan.fused_prefetch ? go(D128{}, On{}) : go(D128{}, Off{}))
                                     : (plan.fused_prefetch ? go(D64{}, On{}) : go(D64{}, Off{}));
  if (e == hipSuccess && n_dec_items > 0) e = launch_decode_merge(cfg, q_start, plan, attn_out, st);
  if (e == hipSuccess && n_pre_items > 0) e = launch_prefill_merge(cfg, q_start, plan, attn_out, st);
  return e;
}

}  // namespace hl
