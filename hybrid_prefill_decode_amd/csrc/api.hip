// Host side of the C ABI: validation on the host mirrors, launch planning, workspace layout and
// the composition of the layer step out of its phases. Nothing here synchronises the device or
// allocates device memory; every launch goes onto the caller's stream.
//
// Step order (one pre-norm decoder layer over the hybrid token matrix):
//   plan -> prep(x) -> QKV GEMM with RoPE + KV-append epilogue
//   -> prefill attention | decode attention + merge -> O GEMM (+x)
//   -> prep(h2) -> gate/up GEMM (SwiGLU) -> down GEMM (+h2)
// prep writes bf16(x * gain) and the RMSNorm row factor, which the next GEMM applies to its fp32
// accumulators (see prep.hip).
// The linear phases see all tokens at once while attention splits by request kind, the
// operator-level split of the "ConfluxServe" summary ("The big picture: what happens inside one
// Transformer layer"), here as one GPU's share.
#include <string.h>

#include <algorithm>
#include <functional>
#include <vector>

#include "common.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct HostPlan {
  int32_t n_dec_units = 0, n_dec_seqs = 0, n_pre_tiles = 0, split_pages = 32;
  int32_t n_pre_merge = 0, n_pre_slots = 0, pre_split = 1 << 30;
  int32_t dec_rank_base[hl::kDecBuckets] = {};  // see hl::Plan
  int32_t dec_lpt = 0;                           // see hl::Plan
  int32_t max_seq_units = 0;                     // see hl::Plan
  bool fused = false;  // prefill and decode attention in one launch
  bool fused_prefetch = false;  // ... whose decode units prefetch their successors
  // workspace byte offsets
  size_t o_dec_units = 0, o_dec_seqs = 0, o_pre_tiles = 0, o_pre_merge = 0, o_pre_po = 0,
         o_pre_ml = 0, o_counters = 0, o_h1 = 0, o_rs = 0, o_pos = 0,
         o_blk = 0, o_cs = 0, o_qlo = 0, o_qrot = 0, o_attn = 0, o_h2 = 0, o_mlp = 0, o_part = 0,
         o_gemm = 0, total = 0;
  size_t gemm_bytes = 0;
};

int check_cfg(const hl_layer_cfg* c) {
  if (!c) return HL_ERR_NULL;
  if (c->head_dim != 64 && c->head_dim != 128) return HL_ERR_SHAPE;
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads) return HL_ERR_SHAPE;
  if (c->n_q_heads / c->n_kv_heads > 16) return HL_ERR_SHAPE;
  if (c->hidden <= 0 || c->hidden % 128) return HL_ERR_SHAPE;
  if (c->d_ff <= 0 || c->d_ff % 64) return HL_ERR_SHAPE;
  if ((c->n_q_heads * c->head_dim) % 64) return HL_ERR_SHAPE;
  if (((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 256) return HL_ERR_SHAPE;
  if (c->block_size != HL_BLOCK_SIZE) return HL_ERR_SHAPE;
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f) || !(c->softmax_scale >= 0.f))
    return HL_ERR_SHAPE;
  // the GEMMs address each operand with 32-bit byte offsets: below 2^31 elements
  const int64_t qkv_cols = (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  const int64_t widest = std::max<int64_t>({qkv_cols, 2 * (int64_t)c->d_ff, c->hidden});
  if (widest * std::max<int64_t>({(int64_t)c->hidden, (int64_t)c->d_ff,
                                  (int64_t)c->n_q_heads * c->head_dim}) > (int64_t)INT32_MAX)
    return HL_ERR_SHAPE;
  return HL_OK;
}

// Descriptor checks that need only the host mirrors.
int check_batch(const hl_batch_desc* b) {
  if (!b || !b->cfg) return HL_ERR_NULL;
  int rc = check_cfg(b->cfg);
  if (rc) return rc;
  if (b->num_seqs < 0 || b->num_tokens < 0) return HL_ERR_DESC;
  if (b->attention < HL_ATTN_AUTO || b->attention > HL_ATTN_SEPARATE) return HL_ERR_DESC;
  if (b->num_seqs == 0) return b->num_tokens == 0 ? HL_OK : HL_ERR_DESC;
  if (!b->h_q_start || !b->h_num_cached || !b->q_start || !b->num_cached) return HL_ERR_NULL;
  if (b->h_q_start[0] != 0) return HL_ERR_DESC;
  for (int s = 0; s < b->num_seqs; ++s) {
    const int64_t qlen = (int64_t)b->h_q_start[s + 1] - b->h_q_start[s];
    if (qlen < 1) return HL_ERR_DESC;
    if (b->h_num_cached[s] < 0) return HL_ERR_DESC;
    if ((int64_t)b->h_num_cached[s] + qlen > (int64_t)1 << 30) return HL_ERR_DESC;
  }
  if (b->h_q_start[b->num_seqs] != b->num_tokens) return HL_ERR_DESC;
  // token rows of every GEMM operand stay within 32-bit byte offsets
  const hl_layer_cfg* c = b->cfg;
  const int64_t row = std::max<int64_t>({(int64_t)c->hidden, (int64_t)c->d_ff,
                                         (int64_t)c->n_q_heads * c->head_dim});
  if ((int64_t)b->num_tokens * row > (int64_t)INT32_MAX) return HL_ERR_DESC;
  return HL_OK;
}

int check_pages(const hl_batch_desc* b, const hl_kv_pages* kv, const hl_block_table* bt) {
  if (!kv || !bt) return HL_ERR_NULL;
  if (!kv->k || !kv->v || !bt->table || !bt->h_table) return HL_ERR_NULL;
  if (!aligned16(kv->k) || !aligned16(kv->v) || !aligned16(bt->table)) return HL_ERR_ALIGN;
  if (kv->num_blocks <= 0 || bt->max_blocks_per_seq <= 0) return HL_ERR_BLOCK;
  for (int s = 0; s < b->num_seqs; ++s) {
    const int64_t kv_len = (int64_t)b->h_num_cached[s] + (b->h_q_start[s + 1] - b->h_q_start[s]);
    const int64_t need = (kv_len + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
    if (need > bt->max_blocks_per_seq) return HL_ERR_BLOCK;
    const int32_t* row = bt->h_table + (size_t)s * bt->max_blocks_per_seq;
    for (int64_t j = 0; j < need; ++j)
      if (row[j] < 0 || (int64_t)row[j] >= kv->num_blocks) return HL_ERR_BLOCK;
  }
  return HL_OK;
}

// Compute units of the current device (queried once per process; every supported device is
// the same part).
int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// Pages per decode work unit. A unit of n pages costs about n + kUnitOverhead page-times (its
// record, query and table reads before the first K/V bytes arrive, the state merge, the partial
// write and its merge read), and two workgroups run per compute unit (the kernel's register
// budget), so `slots` units run at once. With equal-length decodes the units run in whole rounds:
// cost = rounds * (largest unit + overhead). Otherwise the grid drains as a list schedule: cost =
// total work / slots + a tenth of the largest unit (the tail of thousands of dispatched units,
// dealt largest first, is far shorter than a whole unit). The constants come from timing every
// unit size on the 70B (512 decodes log-uniform in 1K..32K) and 14B (96 decodes uniform in
// 2K..8K) batches: the overhead is ~14 page-times. The tail share was a quarter while units ran in
// sequence order; with the largest-first order a tenth picks 681- instead of 511-page units on the
// 70B batch (decode 2974 -> 2962 us) and leaves the 14B one as it was (a twentieth: 2952 us, but
// the 14B batch 6 us slower). Candidates are a
// fixed ladder plus ceil(P_max / u) for small u (which tiles equal lengths exactly); the cheapest
// wins, ties to the larger unit (fewer partials). No sequence may need more than
// kMaxUnitsPerSeq units (its merge weights live in LDS).
int pick_split(const hl_batch_desc* b) {
  constexpr int64_t kUnitOverhead = 14;
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t hkv = b->cfg->n_kv_heads;
  std::vector<int64_t> pages;
  int64_t max_pages = 0, min_pages = INT64_MAX;
  for (int s = 0; s < b->num_seqs; ++s)
    if (b->h_q_start[s + 1] - b->h_q_start[s] == 1) {
      const int64_t p = ((int64_t)b->h_num_cached[s] + HL_BLOCK_SIZE) / HL_BLOCK_SIZE;
      pages.push_back(p);
      max_pages = std::max(max_pages, p);
      min_pages = std::min(min_pages, p);
    }
  if (pages.empty()) return 32;
  const bool uniform = min_pages == max_pages;
  const int64_t sp_min =
      std::max<int64_t>(8, (max_pages + hl::kMaxUnitsPerSeq - 1) / hl::kMaxUnitsPerSeq);
  const int64_t sp_max = std::max<int64_t>(sp_min, std::min<int64_t>(max_pages, 1 << 20));
  std::vector<int64_t> cand = {8,  12,  16,  20,  24,  28,  32,  40,  48,   56,   64,  80,
                               96, 112, 128, 160, 192, 256, 320, 384, 512, 768, 1024};
  for (int64_t u = 1; u <= 64; ++u) cand.push_back((max_pages + u - 1) / u);
  int64_t best_sp = sp_min;
  double best_cost = -1.0;
  for (int64_t sp : cand) {
    sp = std::min(std::max(sp, sp_min), sp_max);
    int64_t units = 0;
    for (int64_t p : pages) units += (p + sp - 1) / sp;
    const int64_t job = std::min(sp, max_pages) + kUnitOverhead;
    double cost;
    if (uniform) {
      cost = (double)((units * hkv + slots - 1) / slots) * (double)job;
    } else {
      double work = 0.0;
      for (int64_t p : pages) work += (double)(p + kUnitOverhead * ((p + sp - 1) / sp));
      cost = work * (double)hkv / (double)slots + 0.1 * (double)job;
    }
    if (best_cost < 0.0 || cost < best_cost - 1e-9 || (cost <= best_cost + 1e-9 && sp > best_sp)) {
      best_cost = cost;
      best_sp = sp;
    }
  }
  return (int)best_sp;
}

// Pages per decode work unit when prefill and decode run in the fused launch: its workers claim
// units dynamically, so units only need to be small enough that every worker gets several (about
// four per worker: the queue then balances the two paths), and large enough to amortise a unit's
// fixed cost. With the units dispatched largest first (`largest_first`) the launch ends on the
// short last units of the sequences whatever the full unit's size, so that size is not capped:
// on the 70B-shaped batch, units of ~1,100 pages instead of 256 cut the launch from 3.06 to
// 2.97 ms (the cap at 512 gave 2.99, 1024 and none 2.97). In sequence order the cap of 256
// pages bounds the tail.
int pick_split_fused(const hl_batch_desc* b, bool largest_first) {
  int64_t total = 0, max_pages = 0;
  for (int s = 0; s < b->num_seqs; ++s)
    if (b->h_q_start[s + 1] - b->h_q_start[s] == 1) {
      const int64_t p = ((int64_t)b->h_num_cached[s] + HL_BLOCK_SIZE) / HL_BLOCK_SIZE;
      total += p;
      max_pages = std::max(max_pages, p);
    }
  const int64_t workers = 2 * (int64_t)device_cus();
  int64_t sp = (total * b->cfg->n_kv_heads + 4 * workers - 1) / (4 * workers);
  sp = std::max<int64_t>(sp, 32);
  if (!largest_first) sp = std::min<int64_t>(sp, 256);
  sp = std::max<int64_t>(sp, (max_pages + hl::kMaxUnitsPerSeq - 1) / hl::kMaxUnitsPerSeq);
  return (int)sp;
}

// Key tiles per prefill work part. Items are (tile or part, query head), two resident per compute
// unit, dealt to the 8 XCDs in (entry, KV head) units (prefill_item_at) and dispatched longest
// first. An item costs a start-up plus one step per key tile; a part of a split tile costs more:
// its fp32 partial rows are written and read back by the merge. A few near-equal items just above
// a multiple of the resident slots leave most slots idle through a last round, and a short chunk
// after a long cached prefix has only Hq items, so the rule compares splits of every tile into
// near-equal parts: for each candidate count of parts of the longest tile it replays the greedy
// longest-first dispatch of one XCD's items over that XCD's slots and keeps the shortest
// makespan (fewer parts on a tie within 2 %), parts never below kMinPart key tiles. A fused
// launch fills the prefill tail with decode units instead, so there tiles are split only when
// the prefill items are fewer than the compute units (measured on the 70B-shaped batch: splitting
// its 256 items costs 1.5 %). The choice depends on the batch's plan only, so every launch of one
// batch (both paths, or either alone) runs the same parts and gives bit-identical rows.
namespace {
constexpr double kItemStart = 2.0;  // start-up of an item, in key-tile steps
constexpr double kPartCost = 6.0;   // partial write + merge read of a split part, in steps
constexpr double kMergeLaunch = 3.0;  // the merge launch that any split adds, in steps

// greedy dispatch of `cost` (in order) over `slots` slots: the makespan
double replay(const std::vector<double>& cost, int slots, std::vector<double>& heap) {
  heap.assign((size_t)slots, 0.0);
  double end = 0.0;
  for (const double c : cost) {
    std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
    heap.back() += c;
    end = std::max(end, heap.back());
    std::push_heap(heap.begin(), heap.end(), std::greater<double>());
  }
  return end;
}
}  // namespace

int pick_pre_split(const hl_batch_desc* b, bool fused) {
  constexpr int kMinPart = 8;
  std::vector<int> tiles;  // key tiles of each prefill tile, in entry order (last tile first)
  int longest = 0;
  for (int s = 0; s < b->num_seqs; ++s) {
    const int n = b->h_q_start[s + 1] - b->h_q_start[s], c = b->h_num_cached[s];
    if (n < 2) continue;
    for (int r0 = ((n - 1) / hl::kPrefillQTile) * hl::kPrefillQTile; r0 >= 0;
         r0 -= hl::kPrefillQTile) {
      tiles.push_back(hl::prefill_key_tiles(c, r0, std::min(hl::kPrefillQTile, n - r0)));
      longest = std::max(longest, tiles.back());
    }
  }
  const int64_t hq = b->cfg->n_q_heads, hkv = b->cfg->n_kv_heads, g = hq / hkv;
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t items = (int64_t)tiles.size() * hq;
  if (tiles.empty() || longest < 2 * kMinPart || items >= 8 * slots) return 1 << 30;
  if (fused) {
    // a fused launch fills the prefill tail with decode units: parts only when there are fewer
    // prefill items than compute units, sized to give every compute unit about one
    const int64_t cus = device_cus();
    if (items >= cus) return 1 << 30;
    int64_t work = 0;
    for (const int nkt : tiles) work += nkt;
    const int64_t split = std::max<int64_t>(kMinPart, (work * hq + cus - 1) / cus);
    return split >= longest ? 1 << 30 : (int)split;
  }
  const int xslots = (int)std::max<int64_t>(1, slots / 8);
  // candidate part counts of the longest tile: 1..8, the counts that fill the slots one to three
  // times over, and the finest split allowed
  std::vector<int> cand = {1, 2, 3, 4, 5, 6, 8, longest / kMinPart};
  for (int64_t k = 1; k <= 3; ++k) cand.push_back((int)((k * slots + items - 1) / items));
  std::vector<double> cost, heap;
  double best = 0.0;
  int best_split = 1 << 30;
  int64_t best_parts = 0;
  for (const int pc : cand) {
    if (pc < 1) continue;
    const int split = (longest + pc - 1) / pc;
    if (split < kMinPart && pc > 1) continue;
    int64_t parts_total = 0;
    for (const int nkt : tiles) parts_total += hl::prefill_parts(nkt, split);
    if (parts_total * hq > 8 * slots && pc > 1) continue;  // the tail is already short
    // section 0 of the dealing: units u = entry * Hkv + k with u % 8 == 0, g items each
    cost.clear();
    int64_t e = 0;
    for (const int nkt : tiles) {
      const int parts = hl::prefill_parts(nkt, split);
      for (int j = 0; j < parts; ++j, ++e) {
        const double steps = (double)((int64_t)(j + 1) * nkt / parts - (int64_t)j * nkt / parts);
        const double c = steps + kItemStart + (parts > 1 ? kPartCost : 0.0);
        for (int64_t k = 0; k < hkv; ++k)
          if ((e * hkv + k) % 8 == 0)
            for (int64_t i = 0; i < g; ++i) cost.push_back(c);
      }
    }
    const double t = replay(cost, xslots, heap) + (parts_total > (int64_t)tiles.size() ? kMergeLaunch : 0.0);
    if (best_parts == 0 || t < 0.98 * best || (t <= best && parts_total < best_parts)) {
      best = t;
      best_split = pc == 1 ? (1 << 30) : split;
      best_parts = parts_total;
    }
  }
  return best_split;
}

void make_plan(const hl_batch_desc* b, HostPlan* p) {
  const hl_layer_cfg& c = *b->cfg;
  *p = HostPlan{};
  // Fused attention pays when a long prefill with many work items can absorb the decode streams
  // (its dynamic queues fill the tail of uneven causal tiles with decode units), or when the
  // decode work is so large that unit granularity does not matter. Otherwise two tuned launches
  // win: the fused kernel's prefill items run slower than the standalone kernel's (the kernel
  // holds both paths' registers), which a short prefill or a little decode work cannot repay.
  // Rule measured on a grid of 8B / 70B batches (prompt chunks of 128..2048 tokens at prefixes
  // 0..8192, 16..256 decodes at 512..8192) and the four large workloads; the estimates use
  // sustained rates of the two kernels (prefill ~0.7 PFLOP/s, decode ~5 TB/s).
  double pre_flops = 0.0, dec_bytes = 0.0;
  int64_t pre_items = 0;
  for (int s = 0; s < b->num_seqs; ++s) {
    const double n = b->h_q_start[s + 1] - b->h_q_start[s], kv = b->h_num_cached[s] + n;
    if (n == 1) {
      dec_bytes += kv * c.n_kv_heads * c.head_dim * 4.0;
    } else {
      pre_flops += 4.0 * c.head_dim * c.n_q_heads * (n * b->h_num_cached[s] + n * (n + 1) / 2);
      pre_items += (int64_t)((n + hl::kPrefillQTile - 1) / hl::kPrefillQTile) * c.n_q_heads;
    }
  }
  const double pre_us = pre_flops / 0.7e9, dec_us = dec_bytes / 5.0e6;  // flop/us, byte/us
  p->fused = pre_flops > 0 && dec_bytes > 0 && pre_us >= 90.0 &&
             ((pre_items >= 512 && dec_us <= 4.0 * pre_us) ||
              (dec_us >= 1000.0 && pre_us >= 0.02 * dec_us));
  if (b->attention == HL_ATTN_FUSED) p->fused = pre_flops > 0 && dec_bytes > 0;
  if (b->attention == HL_ATTN_SEPARATE) p->fused = false;
  // In a fused launch the decode units can start their successor's loads while they drain, which
  // hides most of a unit's start-up but costs the kernel registers that its prefill items then
  // spill: worth it when decode work dominates (measured: the 70B-shaped batch with 512 decodes
  // gains 4 %, prefill-heavy batches lose 5-10 %).
  p->fused_prefetch = p->fused && dec_us >= 4.0 * pre_us;
  p->split_pages = p->fused ? pick_split_fused(b, p->fused_prefetch) : pick_split(b);
  // Decode units largest first (a shorter tail) where decode work decides the launch's length:
  // the separate decode kernel and decode-heavy fused launches (the 70B-shaped batch: -75 us of
  // 3.14 ms). A prefill-heavy fused launch keeps sequence order, which measured ~10 us faster
  // there (its decode units finish long before its prefill items).
  p->dec_lpt = (!p->fused || p->fused_prefetch) ? 1 : 0;
  p->pre_split = pick_pre_split(b, p->fused);
  int64_t last_units[hl::kDecBuckets] = {};
  for (int s = 0; s < b->num_seqs; ++s) {
    const int qlen = b->h_q_start[s + 1] - b->h_q_start[s];
    if (qlen == 1) {
      const int pages = (b->h_num_cached[s] + 1 + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
      const int units = (pages + p->split_pages - 1) / p->split_pages;
      p->n_dec_units += units;
      p->max_seq_units = std::max(p->max_seq_units, units);
      p->n_dec_seqs += 1;
      const int rem = pages % p->split_pages;
      if (rem) ++last_units[hl::dec_bucket(rem, p->split_pages)];
    } else {
      // the plan kernel's count of entries, partial slots and merges (same functions)
      for (int r0 = 0; r0 < qlen; r0 += hl::kPrefillQTile) {
        const int parts = hl::prefill_parts(
            hl::prefill_key_tiles(b->h_num_cached[s], r0, std::min(hl::kPrefillQTile, qlen - r0)),
            p->pre_split);
        p->n_pre_tiles += parts;
        if (parts > 1) {
          p->n_pre_slots += parts;
          p->n_pre_merge += 1;
        }
      }
    }
  }
  // ranks: full units first, then the shorter last units by size class, longest class first
  int64_t rank = p->n_dec_units;
  for (int k = 0; k < hl::kDecBuckets; ++k) rank -= last_units[k];
  for (int k = hl::kDecBuckets - 1; k >= 0; --k) {
    p->dec_rank_base[k] = (int32_t)rank;
    rank += last_units[k];
  }
  const size_t T = (size_t)b->num_tokens;
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t g = (size_t)(c.n_q_heads / c.n_kv_heads);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p->o_counters = take(sizeof(int32_t) * hl::kPlanCounters * hl::kCounterStride);
  p->o_dec_units = take(sizeof(int32_t) * hl::kDecUnitInts * (size_t)p->n_dec_units);
  p->o_dec_seqs = take(sizeof(int32_t) * 3 * (size_t)p->n_dec_seqs);
  p->o_pre_tiles = take(sizeof(int32_t) * hl::kPreEntry * (size_t)p->n_pre_tiles);
  p->o_pre_merge = take(sizeof(int32_t) * 4 * (size_t)p->n_pre_merge);
  const size_t pre_rows = (size_t)p->n_pre_slots * c.n_q_heads * hl::kPrefillQTile;
  p->o_pre_po = take(sizeof(float) * pre_rows * c.head_dim);
  p->o_pre_ml = take(sizeof(float) * 2 * pre_rows);
  p->o_h1 = take(2 * T * c.hidden);
  p->o_rs = take(4 * T);
  p->o_pos = take(4 * T);
  p->o_blk = take(4 * T);
  p->o_cs = take(8 * T * (size_t)(c.head_dim / 2));
  p->o_qrot = take(2 * T * qd);
  p->o_qlo = take(2 * T * qd);
  p->o_attn = take(2 * T * qd);
  p->o_h2 = take(2 * T * c.hidden);
  p->o_mlp = take(2 * T * c.d_ff);
  p->o_part = take(sizeof(float) * (size_t)p->n_dec_units * c.n_kv_heads * g * (c.head_dim + 2));
  p->gemm_bytes = hl::gemm_workspace_bytes(b->num_tokens, c.hidden, c.d_ff, HL_EPI_RESIDUAL);
  p->o_gemm = take(p->gemm_bytes);
  p->total = off;
}

hl::Plan device_plan(const HostPlan& hp, void* ws) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  hl::Plan p;
  p.dec_units = reinterpret_cast<int32_t*>(base + hp.o_dec_units);
  p.dec_seqs = reinterpret_cast<int32_t*>(base + hp.o_dec_seqs);
  p.pre_tiles = reinterpret_cast<int32_t*>(base + hp.o_pre_tiles);
  p.pre_merge = reinterpret_cast<int32_t*>(base + hp.o_pre_merge);
  p.pre_part_o = reinterpret_cast<float*>(base + hp.o_pre_po);
  p.pre_part_ml = reinterpret_cast<float2*>(base + hp.o_pre_ml);
  p.dec_part = reinterpret_cast<float*>(base + hp.o_part);
  p.counters = reinterpret_cast<int32_t*>(base + hp.o_counters);
  p.n_dec_units = hp.n_dec_units;
  p.n_dec_seqs = hp.n_dec_seqs;
  p.n_pre_tiles = hp.n_pre_tiles;
  p.n_pre_merge = hp.n_pre_merge;
  p.split_pages = hp.split_pages;
  for (int k = 0; k < hl::kDecBuckets; ++k) p.dec_rank_base[k] = hp.dec_rank_base[k];
  p.dec_lpt = hp.dec_lpt;
  p.max_seq_units = hp.max_seq_units;
  p.pre_split = hp.pre_split;
  p.fused_prefetch = hp.fused_prefetch;
  return p;
}

// Validation shared by every entry point that takes a batch; fills the host plan.
int prepare(const hl_batch_desc* b, const hl_kv_pages* kv, const hl_block_table* bt,
            HostPlan* hp) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (b->num_seqs == 0) return HL_OK;
  if (!aligned16(b->q_start) || !aligned16(b->num_cached)) return HL_ERR_ALIGN;
  rc = check_pages(b, kv, bt);
  if (rc) return rc;
  make_plan(b, hp);
  if (!b->workspace || b->workspace_bytes < hp->total) return HL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(b->workspace) & (kAlign - 1)) return HL_ERR_ALIGN;
  for (const void* t : {(const void*)b->tap_q_rot, (const void*)b->tap_attn_out,
                        (const void*)b->tap_h2})
    if (t && !aligned16(t)) return HL_ERR_ALIGN;
  return HL_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? HL_OK : HL_ERR_HIP; }

struct Buffers {
  hl_bf16 *h1, *qrot, *qlo, *attn, *h2, *mlp;
  void* gemm_ws;
  size_t gemm_bytes;
  float* rs;
  int32_t *pos, *blk;
  float2* cs;
};

Buffers buffers(const hl_batch_desc* b, const HostPlan& hp) {
  uint8_t* base = static_cast<uint8_t*>(b->workspace);
  Buffers B;
  B.h1 = reinterpret_cast<hl_bf16*>(base + hp.o_h1);
  B.rs = reinterpret_cast<float*>(base + hp.o_rs);
  B.qlo = reinterpret_cast<hl_bf16*>(base + hp.o_qlo);
  B.pos = reinterpret_cast<int32_t*>(base + hp.o_pos);
  B.blk = reinterpret_cast<int32_t*>(base + hp.o_blk);
  B.cs = reinterpret_cast<float2*>(base + hp.o_cs);
  B.qrot = b->tap_q_rot ? b->tap_q_rot : reinterpret_cast<hl_bf16*>(base + hp.o_qrot);
  B.attn = b->tap_attn_out ? b->tap_attn_out : reinterpret_cast<hl_bf16*>(base + hp.o_attn);
  B.h2 = b->tap_h2 ? b->tap_h2 : reinterpret_cast<hl_bf16*>(base + hp.o_h2);
  B.mlp = reinterpret_cast<hl_bf16*>(base + hp.o_mlp);
  B.gemm_ws = base + hp.o_gemm;
  B.gemm_bytes = hp.gemm_bytes;
  return B;
}

hl::GemmEpi plain_epi(int kind, const hl_bf16* residual, const float* row_scale) {
  hl::GemmEpi e{};
  e.kind = kind;
  e.residual = residual;
  e.row_scale = row_scale;
  return e;
}

// prep(x) + QKV GEMM with the RoPE / KV-append epilogue; with `plan`, the prep pass also builds
// the attention work lists.
int run_qkv(const hl_batch_desc* b, const hl_weights* w, hl_bf16* q_rot, const hl_kv_pages* kv,
            const hl_block_table* bt, const Buffers& B, const hl::Plan* plan = nullptr) {
  const hl_layer_cfg& c = *b->cfg;
  hipStream_t st = static_cast<hipStream_t>(b->stream);
  hl::TokenInfo ti{b->q_start, b->num_cached, b->num_seqs, bt->table, bt->max_blocks_per_seq,
                   kv->num_blocks, c.head_dim, c.rope_theta, B.pos, B.blk, B.cs};
  int rc = hip_rc(hl::launch_prep(b->x, w->attn_norm, B.h1, B.rs, b->num_tokens, c.hidden,
                                  c.rms_eps, &ti, st, plan));
  if (rc) return rc;
  hl::GemmEpi e = plain_epi(hl::kEpiRopeAppend, nullptr, B.rs);
  e.n_q_heads = c.n_q_heads;
  e.n_kv_heads = c.n_kv_heads;
  e.head_dim = c.head_dim;
  e.q_rot = q_rot;
  e.q_lo = B.qlo;
  e.kpool = kv->k;
  e.vpool = kv->v;
  e.tok_pos = B.pos;
  e.tok_blk = B.blk;
  e.rope_cs = B.cs;
  const int qkv_cols = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  return hip_rc(hl::launch_gemm(B.h1, w->w_qkv, nullptr, b->num_tokens, qkv_cols, c.hidden, e,
                                B.gemm_ws, B.gemm_bytes, st));
}

// plan_built: the work lists are already in the workspace (built by the step's prep pass).
int run_attention(const hl_batch_desc* b, const hl_bf16* q_rot, const hl_bf16* q_lo,
                  const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out,
                  const HostPlan& hp, bool do_prefill, bool do_decode, bool plan_built = false,
                  uint64_t* trace = nullptr) {
  hipStream_t st = static_cast<hipStream_t>(b->stream);
  hl::Plan dp = device_plan(hp, b->workspace);
  dp.trace = trace;
  int rc = plan_built ? HL_OK
                      : hip_rc(hl::launch_plan(b->q_start, b->num_cached, b->num_seqs, bt->table,
                                          bt->max_blocks_per_seq, dp, st));
  if (rc) return rc;
  if (do_prefill && do_decode && hp.fused) {
    // both paths in one fused launch: prefill and decode overlap on every compute unit
    return hip_rc(hl::launch_hybrid_attention(*b->cfg, b->q_start, b->num_cached, q_rot, q_lo,
                                              kv->k, kv->v, kv->num_blocks, bt->table,
                                              bt->max_blocks_per_seq, dp, device_cus(), attn_out,
                                              st));
  }
  if (do_prefill) {
    rc = hip_rc(hl::launch_prefill_attention(*b->cfg, b->q_start, b->num_cached, q_rot, kv->k,
                                             kv->v, kv->num_blocks, bt->table,
                                             bt->max_blocks_per_seq, dp, attn_out, st));
    if (rc) return rc;
  }
  if (do_decode) {
    rc = hip_rc(hl::launch_decode_attention(*b->cfg, b->q_start, b->num_cached, q_rot, q_lo, kv->k,
                                            kv->v, kv->num_blocks, bt->table,
                                            bt->max_blocks_per_seq, dp, device_cus(), attn_out,
                                            st));
  }
  return rc;
}

int check_weights(const hl_weights* w) {
  if (!w) return HL_ERR_NULL;
  if (!w->attn_norm || !w->w_qkv || !w->w_o || !w->mlp_norm || !w->w_gate_up || !w->w_down)
    return HL_ERR_NULL;
  for (const void* p : {(const void*)w->attn_norm, (const void*)w->w_qkv, (const void*)w->w_o,
                        (const void*)w->mlp_norm, (const void*)w->w_gate_up,
                        (const void*)w->w_down})
    if (!aligned16(p)) return HL_ERR_ALIGN;
  return HL_OK;
}

// The layer on a validated batch and plan.
int run_layer(const hl_batch_desc* batch, const hl_weights* w, hl_kv_pages* kv,
              const hl_block_table* bt, const HostPlan& hp, hl_bf16* out) {
  const hl_layer_cfg& c = *batch->cfg;
  const int T = batch->num_tokens;
  const int qd = c.n_q_heads * c.head_dim;
  hipStream_t st = static_cast<hipStream_t>(batch->stream);
  const Buffers B = buffers(batch, hp);
  int rc;
  const hl::Plan dp = device_plan(hp, batch->workspace);
  // the caller's phase marks (hl_batch_desc::events), if any
  auto mark = [&](int i) -> int {
    if (!batch->events || !batch->events[i]) return HL_OK;
    return hipEventRecord(static_cast<hipEvent_t>(batch->events[i]), st) == hipSuccess
               ? HL_OK
               : HL_ERR_HIP;
  };
  if ((rc = mark(0))) return rc;
  if ((rc = run_qkv(batch, w, B.qrot, kv, bt, B, &dp))) return rc;
  if ((rc = mark(1))) return rc;
  if ((rc = run_attention(batch, B.qrot, B.qlo, kv, bt, B.attn, hp, true, true, true))) return rc;
  if ((rc = mark(2))) return rc;
  if ((rc = hip_rc(hl::launch_gemm(B.attn, w->w_o, B.h2, T, c.hidden, qd,
                                   plain_epi(HL_EPI_RESIDUAL, batch->x, nullptr), B.gemm_ws,
                                   B.gemm_bytes, st))))
    return rc;
  if ((rc = mark(3))) return rc;
  if ((rc = hip_rc(hl::launch_prep(B.h2, w->mlp_norm, B.h1, B.rs, T, c.hidden, c.rms_eps,
                                   nullptr, st))))
    return rc;
  if ((rc = mark(4))) return rc;
  if ((rc = hip_rc(hl::launch_gemm(B.h1, w->w_gate_up, B.mlp, T, 2 * c.d_ff, c.hidden,
                                   plain_epi(HL_EPI_SWIGLU, nullptr, B.rs), B.gemm_ws,
                                   B.gemm_bytes, st))))
    return rc;
  if ((rc = mark(5))) return rc;
  if ((rc = hip_rc(hl::launch_gemm(B.mlp, w->w_down, out, T, c.hidden, c.d_ff,
                                   plain_epi(HL_EPI_RESIDUAL, B.h2, nullptr), B.gemm_ws,
                                   B.gemm_bytes, st))))
    return rc;
  return mark(6);
}

// Model workspace: the step's workspace, then two [T, H] residual-stream buffers, the last row of
// each sequence and its gain-scaled copy ([S, H] each), and the final norm's row factors [S].
struct ModelLayout {
  size_t o_x0, o_x1, o_rows, o_rows_g, o_rs, total;
};
ModelLayout model_layout(const hl_batch_desc* b, size_t step_bytes) {
  auto up = [](size_t v) { return (v + kAlign - 1) / kAlign * kAlign; };
  const size_t T = b->num_tokens, S = b->num_seqs, H = b->cfg->hidden;
  ModelLayout m;
  m.o_x0 = up(step_bytes);
  m.o_x1 = m.o_x0 + up(T * H * 2);
  m.o_rows = m.o_x1 + up(T * H * 2);
  m.o_rows_g = m.o_rows + up(S * H * 2);
  m.o_rs = m.o_rows_g + up(S * H * 2);
  m.total = m.o_rs + up(S * 4);
  return m;
}

}  // namespace

extern "C" {

int hl_version(void) { return HL_VERSION; }

const char* hl_strerror(int code) {
  switch (code) {
    case HL_OK: return "ok";
    case HL_ERR_NULL: return "a required pointer is NULL";
    case HL_ERR_SHAPE: return "unsupported layer dimensions";
    case HL_ERR_DESC: return "invalid batch descriptor (q_start / num_cached / num_tokens)";
    case HL_ERR_BLOCK: return "block table too short or block id out of range";
    case HL_ERR_ALIGN: return "device pointer not 16-byte aligned (workspace: 256-byte)";
    case HL_ERR_WORKSPACE: return "workspace missing or too small";
    case HL_ERR_HIP: return "HIP kernel launch failed";
    case HL_ERR_ARG: return "invalid argument";
    default: return "unknown error code";
  }
}

int hl_attention_plan(const hl_batch_desc* batch, int32_t* fused, int32_t* split_pages,
                      int32_t* decode_units, int32_t* prefill_parts, int32_t* prefill_split,
                      int32_t* prefill_merges) {
  if (!fused || !split_pages || !decode_units || !prefill_parts || !prefill_split ||
      !prefill_merges)
    return HL_ERR_NULL;
  int rc = check_batch(batch);
  if (rc) return rc;
  HostPlan hp;
  if (batch->num_seqs > 0) make_plan(batch, &hp);
  *fused = hp.fused ? (hp.fused_prefetch ? 2 : 1) : 0;
  *split_pages = hp.split_pages;
  *decode_units = hp.n_dec_units;
  *prefill_parts = hp.n_pre_tiles;
  *prefill_split = hp.pre_split;
  *prefill_merges = hp.n_pre_merge;
  return HL_OK;
}

int hl_workspace_bytes(const hl_batch_desc* batch, size_t* bytes) {
  if (!bytes) return HL_ERR_NULL;
  int rc = check_batch(batch);
  if (rc) return rc;
  HostPlan hp;
  if (batch->num_seqs == 0) {
    *bytes = 0;
    return HL_OK;
  }
  make_plan(batch, &hp);
  *bytes = hp.total;
  return HL_OK;
}

int hl_rmsnorm(const hl_bf16* x, const hl_bf16* gain, hl_bf16* y, int32_t rows, int32_t cols,
               float eps, void* stream) {
  if (!x || !gain || !y) return HL_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 8 || !(eps >= 0.f)) return HL_ERR_ARG;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(y)) return HL_ERR_ALIGN;
  return hip_rc(hl::launch_rmsnorm(x, gain, y, rows, cols, eps, static_cast<hipStream_t>(stream)));
}

int hl_gemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t epilogue, size_t* bytes) {
  if (!bytes) return HL_ERR_NULL;
  *bytes = hl::gemm_workspace_bytes(m, n, k, epilogue);
  return HL_OK;
}

int hl_gemm_tile_choice(int32_t m, int32_t n, int32_t k, int32_t epilogue, int32_t with_workspace,
                        int32_t qkv_head_dim, int32_t* tile_m, int32_t* tile_n, int32_t* stream_k,
                        int32_t* splits) {
  if (!tile_m || !tile_n || !stream_k || !splits) return HL_ERR_NULL;
  *splits = 0;
  if (epilogue != HL_EPI_NONE && epilogue != HL_EPI_RESIDUAL && epilogue != HL_EPI_SWIGLU)
    return HL_ERR_ARG;
  if (m < 0 || n <= 0 || k <= 0 || k % 64 || n % 128) return HL_ERR_ARG;
  if (qkv_head_dim != 0 && qkv_head_dim != 64 && qkv_head_dim != 128) return HL_ERR_ARG;
  if (with_workspace && hl::use_skinny(m, n, k, hl::gemm_workspace_bytes(m, n, k, epilogue))) {
    *tile_m = 16 * ((m + 15) / 16);
    *tile_n = 64;
    *stream_k = 2;
    return HL_OK;
  }
  int sched = 0;
  if (with_workspace)
    sched = ((qkv_head_dim || epilogue == HL_EPI_SWIGLU)
                 ? hl::kSchedSplitK
                 : hl::kSchedStreamK | hl::kSchedSplitK | hl::kSchedWideSplit) |
            hl::kSchedTail;
  if (epilogue == HL_EPI_SWIGLU && !qkv_head_dim) sched |= hl::kSchedSwigluTiles;
  const hl::TileChoice tc = hl::choose_tiles(m, n, k, sched, qkv_head_dim ? qkv_head_dim : 1);
  *tile_m = tc.bm;
  *tile_n = tc.bn;
  *stream_k = tc.sk ? 1 : (tc.splits >= 2 ? (tc.tail ? 4 : 3) : 0);
  *splits = tc.splits >= 2 ? tc.splits : 0;
  return HL_OK;
}

int hl_rms_scale(const hl_bf16* x, const hl_bf16* gain, hl_bf16* xg, float* row_scale,
                 int32_t rows, int32_t cols, float eps, void* stream) {
  if (!x || !gain || !xg || !row_scale) return HL_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 8 || !(eps >= 0.f)) return HL_ERR_ARG;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(xg)) return HL_ERR_ALIGN;
  return hip_rc(hl::launch_prep(x, gain, xg, row_scale, rows, cols, eps, nullptr,
                                static_cast<hipStream_t>(stream)));
}

int check_gemm_args(const hl_bf16* a, const hl_bf16* w, const hl_bf16* c,
                    const hl_bf16* residual, int32_t m, int32_t n, int32_t k, int32_t epilogue) {
  if (!a || !w || !c) return HL_ERR_NULL;
  if (epilogue != HL_EPI_NONE && epilogue != HL_EPI_RESIDUAL && epilogue != HL_EPI_SWIGLU)
    return HL_ERR_ARG;
  if (epilogue == HL_EPI_RESIDUAL && !residual) return HL_ERR_NULL;
  if (m < 0 || n <= 0 || k <= 0 || k % 64 || n % 128) return HL_ERR_ARG;
  if ((int64_t)m * k > (int64_t)INT32_MAX || (int64_t)n * k > (int64_t)INT32_MAX) return HL_ERR_ARG;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c) || (residual && !aligned16(residual)))
    return HL_ERR_ALIGN;
  return HL_OK;
}

int hl_gemm_bf16_nt(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, const hl_bf16* residual,
                    const float* row_scale, int32_t m, int32_t n, int32_t k, int32_t epilogue,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_gemm_args(a, w, c, residual, m, n, k, epilogue);
  if (rc) return rc;
  return hip_rc(hl::launch_gemm(a, w, c, m, n, k, plain_epi(epilogue, residual, row_scale),
                                workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

int hl_gemm_bf16_nt_tiled(const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                          const hl_bf16* residual, const float* row_scale, int32_t m, int32_t n,
                          int32_t k, int32_t epilogue, int32_t tile_m, int32_t tile_n,
                          int32_t stream_k, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const int rc = check_gemm_args(a, w, c, residual, m, n, k, epilogue);
  if (rc) return rc;
  if (!hl::gemm_tile_supported(tile_m, tile_n, epilogue, stream_k) || n % tile_n) return HL_ERR_ARG;
  if (stream_k == -1 || stream_k < -8) return HL_ERR_ARG;
  if (stream_k && (!workspace || workspace_bytes < hl::gemm_workspace_bytes(m, n, k, epilogue)))
    return HL_ERR_ARG;
  // 1: stream-K (plain / residual); s >= 2: split-K into s K ranges; -s (2 <= s <= 8): one tile
  // per workgroup, the tiles past the last full round split into s K ranges
  if (stream_k == 1 && epilogue == HL_EPI_SWIGLU) return HL_ERR_ARG;
  if (stream_k >= 2 && (stream_k > k / 64 || !hl::gemm_split_fits(m, n, tile_m, tile_n, stream_k)))
    return HL_ERR_ARG;
  if (stream_k <= -2 && (-stream_k > k / 64 || !hl::gemm_tail_fits(m, n, tile_m, tile_n, -stream_k)))
    return HL_ERR_ARG;
  if (m == 0) return HL_OK;
  const hl::TileChoice tc{tile_m, tile_n, stream_k == 1,
                          stream_k >= 2 ? stream_k : (stream_k <= -2 ? -stream_k : 0),
                          stream_k <= -2};
  return hip_rc(hl::launch_gemm_tiles(a, w, c, m, n, k, plain_epi(epilogue, residual, row_scale),
                                      tc, workspace, static_cast<hipStream_t>(stream)));
}

// Host checks of a KV span (nothing is launched on failure).
int check_span(const hl_kv_span* s, const hl_kv_pages* kv, const void* buf) {
  if (!s || !kv || !buf) return HL_ERR_NULL;
  if (s->n_kv_heads <= 0 || (s->head_dim != 64 && s->head_dim != 128)) return HL_ERR_ARG;
  if (s->num_layers <= 0 || s->layer < 0 || s->layer >= s->num_layers) return HL_ERR_ARG;
  if (s->start < 0 || s->count < 0 || s->table_len < 0) return HL_ERR_ARG;
  if ((int64_t)s->start + s->count > (int64_t)HL_BLOCK_SIZE * s->table_len) return HL_ERR_ARG;
  if (s->count == 0) return HL_OK;
  if (!s->table || !s->h_table || !kv->k || !kv->v) return HL_ERR_NULL;
  if (!aligned16(kv->k) || !aligned16(kv->v) || !aligned16(buf)) return HL_ERR_ALIGN;
  const int first = s->start / HL_BLOCK_SIZE, last = (s->start + s->count - 1) / HL_BLOCK_SIZE;
  for (int j = first; j <= last; ++j)
    if (s->h_table[j] < 0 || s->h_table[j] >= kv->num_blocks) return HL_ERR_BLOCK;
  return HL_OK;
}

int hl_kv_export(const hl_kv_span* span, const hl_kv_pages* kv, hl_bf16* dst) {
  const int rc = check_span(span, kv, dst);
  if (rc || span->count == 0) return rc;
  return hip_rc(hl::launch_kv_span(*span, *kv, dst, true));
}

int hl_kv_import(const hl_kv_span* span, const hl_bf16* src, hl_kv_pages* kv) {
  const int rc = check_span(span, kv, src);
  if (rc || span->count == 0) return rc;
  return hip_rc(hl::launch_kv_span(*span, *kv, const_cast<hl_bf16*>(src), false));
}

int hl_rope_kv_append(const hl_batch_desc* batch, const hl_bf16* qkv, hl_bf16* q_rot,
                      hl_kv_pages* kv, const hl_block_table* bt) {
  HostPlan hp;
  int rc = check_batch(batch);
  if (rc) return rc;
  if (batch->num_seqs == 0) return HL_OK;
  if (!qkv || !q_rot) return HL_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(q_rot)) return HL_ERR_ALIGN;
  rc = check_pages(batch, kv, bt);
  if (rc) return rc;
  (void)hp;
  return hip_rc(hl::launch_rope_append(*batch->cfg, batch->num_seqs, batch->num_tokens,
                                       batch->q_start, batch->num_cached, qkv, q_rot, kv->k,
                                       kv->v, kv->num_blocks, bt->table, bt->max_blocks_per_seq,
                                       static_cast<hipStream_t>(batch->stream)));
}

int hl_qkv_rope_append(const hl_batch_desc* batch, const hl_weights* w, hl_bf16* q_rot,
                       hl_kv_pages* kv, const hl_block_table* bt) {
  HostPlan hp;
  int rc = prepare(batch, kv, bt, &hp);
  if (rc) return rc;
  if (batch->num_seqs == 0) return HL_OK;
  if (!w || !w->attn_norm || !w->w_qkv || !q_rot || !batch->x) return HL_ERR_NULL;
  if (!aligned16(w->attn_norm) || !aligned16(w->w_qkv) || !aligned16(q_rot) ||
      !aligned16(batch->x))
    return HL_ERR_ALIGN;
  return run_qkv(batch, w, q_rot, kv, bt, buffers(batch, hp));
}

static int attention_entry(const hl_batch_desc* batch, const hl_bf16* q_rot,
                           const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out,
                           bool pre, bool dec) {
  HostPlan hp;
  int rc = prepare(batch, kv, bt, &hp);
  if (rc) return rc;
  if (batch->num_seqs == 0) return HL_OK;
  if (!q_rot || !attn_out) return HL_ERR_NULL;
  if (!aligned16(q_rot) || !aligned16(attn_out)) return HL_ERR_ALIGN;
  return run_attention(batch, q_rot, nullptr, kv, bt, attn_out, hp, pre, dec);
}

int hl_attention(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_kv_pages* kv,
                 const hl_block_table* bt, hl_bf16* attn_out) {
  return attention_entry(batch, q_rot, kv, bt, attn_out, true, true);
}
int hl_prefill_attention(const hl_batch_desc* batch, const hl_bf16* q_rot,
                         const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out) {
  return attention_entry(batch, q_rot, kv, bt, attn_out, true, false);
}
int hl_decode_attention(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_kv_pages* kv,
                        const hl_block_table* bt, hl_bf16* attn_out) {
  return attention_entry(batch, q_rot, kv, bt, attn_out, false, true);
}

int hl_attention_build_lists(const hl_batch_desc* batch, const hl_kv_pages* kv,
                             const hl_block_table* bt) {
  HostPlan hp;
  int rc = prepare(batch, kv, bt, &hp);
  if (rc || batch->num_seqs == 0) return rc;
  const hl::Plan dp = device_plan(hp, batch->workspace);
  return hip_rc(hl::launch_plan(batch->q_start, batch->num_cached, batch->num_seqs, bt->table,
                                bt->max_blocks_per_seq, dp, static_cast<hipStream_t>(batch->stream)));
}

static int attention_run(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_bf16* q_lo,
                         const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out,
                         int32_t paths, uint64_t* trace, size_t trace_entries, bool traced) {
  if (paths < 1 || paths > 3) return HL_ERR_ARG;
  HostPlan hp;
  int rc = prepare(batch, kv, bt, &hp);
  if (rc || batch->num_seqs == 0) return rc;
  if (!q_rot || !attn_out) return HL_ERR_NULL;
  if (!aligned16(q_rot) || !aligned16(attn_out) || (q_lo && !aligned16(q_lo))) return HL_ERR_ALIGN;
  if (traced) {
    const size_t items = (size_t)hp.n_pre_tiles * batch->cfg->n_q_heads +
                         (size_t)hp.n_dec_units * batch->cfg->n_kv_heads;
    if (!trace) return HL_ERR_NULL;
    if (!aligned16(trace)) return HL_ERR_ALIGN;
    if (trace_entries < 3 * items) return HL_ERR_ARG;
  }
  return run_attention(batch, q_rot, q_lo, kv, bt, attn_out, hp, (paths & 1) != 0,
                       (paths & 2) != 0, true, traced ? trace : nullptr);
}

int hl_attention_run(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_bf16* q_lo,
                     const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out,
                     int32_t paths) {
  return attention_run(batch, q_rot, q_lo, kv, bt, attn_out, paths, nullptr, 0, false);
}

int hl_attention_run_traced(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_bf16* q_lo,
                            const hl_kv_pages* kv, const hl_block_table* bt, hl_bf16* attn_out,
                            int32_t paths, uint64_t* trace, size_t trace_entries) {
  return attention_run(batch, q_rot, q_lo, kv, bt, attn_out, paths, trace, trace_entries, true);
}

int hl_trace_clock_khz(int32_t* khz) {
  if (!khz) return HL_ERR_NULL;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return HL_ERR_HIP;
  *khz = rate;
  return HL_OK;
}

int hybrid_layer_step(const hl_batch_desc* batch, const hl_weights* w, hl_kv_pages* kv,
                      const hl_block_table* bt, hl_bf16* out) {
  HostPlan hp;
  int rc = prepare(batch, kv, bt, &hp);
  if (rc) return rc;
  if (batch->num_seqs == 0) return HL_OK;
  if (!out || !batch->x) return HL_ERR_NULL;
  if (!aligned16(batch->x) || !aligned16(out)) return HL_ERR_ALIGN;
  if ((rc = check_weights(w))) return rc;
  if ((const void*)out == (const void*)batch->x) return HL_ERR_ARG;
  return run_layer(batch, w, kv, bt, hp, out);
}

int hl_model_workspace_bytes(const hl_model* m, const hl_batch_desc* batch, size_t* bytes) {
  if (!m || !batch || !bytes) return HL_ERR_NULL;
  int rc = check_batch(batch);
  if (rc) return rc;
  HostPlan hp;
  if (batch->num_seqs > 0) make_plan(batch, &hp);
  *bytes = model_layout(batch, batch->num_seqs > 0 ? hp.total : 0).total;
  return HL_OK;
}

int hl_model_step(const hl_model* m, const hl_batch_desc* batch, const int32_t* tokens,
                  const int32_t* h_tokens, const hl_block_table* bt, hl_bf16* hidden_out,
                  hl_bf16* logits, int32_t* next_tokens) {
  if (!m || !batch) return HL_ERR_NULL;
  int rc = check_batch(batch);
  if (rc) return rc;
  if (batch->num_seqs == 0) return HL_OK;
  if (m->num_layers < 1 || m->vocab <= 0 || m->vocab % 128) return HL_ERR_ARG;
  if ((int64_t)m->vocab * batch->cfg->hidden > (int64_t)INT32_MAX) return HL_ERR_ARG;
  if (!m->embed || !m->final_norm || !m->lm_head || !m->layers || !m->kv) return HL_ERR_NULL;
  if (!tokens || !h_tokens || !logits || !next_tokens) return HL_ERR_NULL;
  for (const void* p : {(const void*)m->embed, (const void*)m->final_norm,
                        (const void*)m->lm_head, (const void*)logits, (const void*)tokens,
                        (const void*)next_tokens})
    if (!aligned16(p)) return HL_ERR_ALIGN;
  if (hidden_out && !aligned16(hidden_out)) return HL_ERR_ALIGN;
  for (int t = 0; t < batch->num_tokens; ++t)
    if (h_tokens[t] < 0 || h_tokens[t] >= m->vocab) return HL_ERR_ARG;
  for (int l = 0; l < m->num_layers; ++l) {
    if ((rc = check_weights(&m->layers[l]))) return rc;
    if (!m->kv[l].k || !m->kv[l].v) return HL_ERR_NULL;
    if (m->kv[l].num_blocks != m->kv[0].num_blocks) return HL_ERR_ARG;
  }
  // plan once for every layer (same batch, same table, pools of one size); the step's own
  // workspace sits first in the model workspace
  HostPlan hp;
  hl_batch_desc inner = *batch;
  if (!batch->workspace) return HL_ERR_WORKSPACE;
  make_plan(batch, &hp);
  const ModelLayout ml = model_layout(batch, hp.total);
  if (batch->workspace_bytes < ml.total) return HL_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(batch->workspace);
  inner.workspace_bytes = hp.total;
  inner.x = reinterpret_cast<hl_bf16*>(base + ml.o_x0);
  inner.tap_q_rot = inner.tap_attn_out = inner.tap_h2 = nullptr;  // per-layer tensors: not kept
  inner.events = nullptr;                                           // phase marks: one layer only
  if ((rc = prepare(&inner, &m->kv[0], bt, &hp))) return rc;

  const hl_layer_cfg& c = *batch->cfg;
  const int T = batch->num_tokens, S = batch->num_seqs, H = c.hidden;
  hipStream_t st = static_cast<hipStream_t>(batch->stream);
  hl_bf16* xa = reinterpret_cast<hl_bf16*>(base + ml.o_x0);
  hl_bf16* xb = reinterpret_cast<hl_bf16*>(base + ml.o_x1);
  if ((rc = hip_rc(hl::launch_embed(tokens, m->embed, xa, T, H, m->vocab, st)))) return rc;
  for (int l = 0; l < m->num_layers; ++l) {
    hl_bf16* dst = (l == m->num_layers - 1 && hidden_out) ? hidden_out : xb;
    inner.x = xa;
    if ((rc = run_layer(&inner, &m->layers[l], &m->kv[l], bt, hp, dst))) return rc;
    xb = xa;
    xa = dst;
  }
  // logits of the last row of every sequence: final RMSNorm as a row factor into the LM head
  hl_bf16* rows = reinterpret_cast<hl_bf16*>(base + ml.o_rows);
  hl_bf16* rows_g = reinterpret_cast<hl_bf16*>(base + ml.o_rows_g);
  float* rrs = reinterpret_cast<float*>(base + ml.o_rs);
  const Buffers B = buffers(&inner, hp);
  if ((rc = hip_rc(hl::launch_last_rows(batch->q_start, xa, rows, S, H, st)))) return rc;
  if ((rc = hip_rc(hl::launch_prep(rows, m->final_norm, rows_g, rrs, S, H, c.rms_eps, nullptr, st))))
    return rc;
  if ((rc = hip_rc(hl::launch_gemm(rows_g, m->lm_head, logits, S, m->vocab, H,
                                   plain_epi(HL_EPI_NONE, nullptr, rrs), B.gemm_ws, B.gemm_bytes,
                                   st))))
    return rc;
  return hip_rc(hl::launch_argmax(logits, S, m->vocab, next_tokens, st));
}

}  // extern "C"
