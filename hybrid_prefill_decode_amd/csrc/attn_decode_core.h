// One split-KV decode work item (a run of pages of one decode sequence, one KV head), run by the
// persistent attention workers (attention_hybrid.hip: the fused prefill + decode launch and the
// decode-only launch). The method and the design are described in attention_decode.hip.
//
// With PREFETCH, a persistent worker running decode items back to back has each wave start its
// part of the next item while the current one drains: near the end of its pages the wave reads
// the workgroup's next item (claimed by thread 0 when the current item started and published in
// LDS), loads that item's record and, in its last page pair, issues the loads of the next item's
// first page pair; the next item's query follows the last product. The chain record -> table ->
// K/V that otherwise opens every item (several dependent memory latencies, about 11 us per item
// under full load) then overlaps the previous item's streaming.
#pragma once
#include "common.h"

namespace hl {
namespace decode {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTickPending = -2;  // DecodeLds::tick before the workgroup's next item is known

struct DecodeArgs {
  const int32_t* q_start;
  const int32_t* num_cached;
  const hl_bf16* q_rot;
  const hl_bf16* q_lo;  // may be null
  const hl_bf16* kpool;
  const hl_bf16* vpool;
  long long num_blocks;
  const int32_t* table;
  int max_blocks;
  const int32_t* units;     // [n][kDecUnitInts]: the units' records (Plan::dec_units)
  const int32_t* dec_seqs;  // [n][3]: (sequence, first unit, unit count)
  int split_pages;
  int Hq, Hkv;
  float scale_log2;
  float* part;
  hl_bf16* attn_out;
  int n_items;      // decode items (units x KV heads)
  int lpt;          // unit records in largest-first dispatch order (Plan::dec_lpt)
};

// LDS of one work item: the waves' (o, m, l) states before they are combined, and the
// workgroup's next decode item (thread 0 writes it once claimed; -1 if there is none).
template <int D>
struct DecodeLds {
  float o[kWaves][D][16];
  float m[kWaves][16];
  float l[kWaves][16];
  int tick;
};

// K/V fragments of one page pair of one wave.
template <int D>
struct Pair {
  u32x4 k[2][D / 32];
  u32x2 v[2][D / 16];
};

// A unit's record (Plan::dec_units).
struct UnitRec {
  int s, pg0, nu, row, kv_len, slot;
};
HL_DEV UnitRec unit_rec(const int32_t* __restrict__ units, int unit) {
  const int32_t* r = units + (size_t)kDecUnitInts * unit;
  const u32x4 a = *reinterpret_cast<const u32x4*>(r);
  const u32x4 b = *reinterpret_cast<const u32x4*>(r + 4);
  // wave-uniform values: scalar registers
  return UnitRec{__builtin_amdgcn_readfirstlane((int)a[0]), __builtin_amdgcn_readfirstlane((int)a[1]),
                 __builtin_amdgcn_readfirstlane((int)a[3]), __builtin_amdgcn_readfirstlane((int)b[0]),
                 __builtin_amdgcn_readfirstlane((int)b[1]), __builtin_amdgcn_readfirstlane((int)b[2])};
}
// block ids of the unit's pages first + 2 wave and first + 2 wave + 1, from the record
HL_DEV void unit_first_pair(const int32_t* __restrict__ units, int unit, int wave, int* blk) {
  const u32x2 v =
      *reinterpret_cast<const u32x2*>(units + (size_t)kDecUnitInts * unit + 8 + 2 * wave);
  blk[0] = __builtin_amdgcn_readfirstlane((int)v[0]);
  blk[1] = __builtin_amdgcn_readfirstlane((int)v[1]);
}

// What a wave carries from one decode item into the workgroup's next: that item (-1: nothing
// prefetched), its record, its query fragments, and its first page pair (loading) with block ids.
template <int D>
struct Carry {
  int item;
  bool has_pair;
  UnitRec rec;
  int blk[2];
  u32x4 qf[D / 32], ql[D / 32];
  Pair<D> first;
};

// Decode item `item` (unit position * Hkv + KV head). Every thread of a kThreads-thread workgroup
// calls it. `cy` holds what the previous item prefetched (used when cy.item == item) and receives
// the prefetch of the next item. Consecutive items of one workgroup must be separated by a barrier
// (the LDS is reused). Returns the item's index in sequence order (partial slot * Hkv + KV head),
// which the work-item trace records are indexed by.
template <int D, bool PREFETCH>
HL_DEV int decode_item(const DecodeArgs& a, int item, DecodeLds<D>& L, Carry<D>& cy) {
  const hl_bf16* __restrict__ q_rot = a.q_rot;
  const hl_bf16* __restrict__ q_lo = a.q_lo;
  const hl_bf16* __restrict__ kpool = a.kpool;
  const hl_bf16* __restrict__ vpool = a.vpool;
  const long long num_blocks = a.num_blocks;
  const int split_pages = a.split_pages, Hq = a.Hq, Hkv = a.Hkv;
  const float scale_log2 = a.scale_log2;
  float* __restrict__ part = a.part;
  hl_bf16* __restrict__ attn_out = a.attn_out;
  auto& sh_o = L.o;
  auto& sh_m = L.m;
  auto& sh_l = L.l;
  const int g = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4;   // lane group 0..3
  const int col = lane & 15;  // S^T / O^T column = query head within the group
  const size_t page_elems = (size_t)HL_BLOCK_SIZE * D;
  const bool two_part = q_lo != nullptr;
  const int unit = item / Hkv, kvh = item - unit * Hkv;
  auto pages_end = [&](const UnitRec& r) {
    return min(r.pg0 + split_pages, (r.kv_len + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE);
  };

  // Q^T operand: lane (lg, col) holds head col, d = 32 ks + 8 lg .. +7
  auto load_q = [&](int row, int kh, u32x4 (&qf)[D / 32], u32x4 (&ql)[D / 32]) {
    const bool ok = col < g;
    const size_t off = ((size_t)row * Hq + kh * g + (ok ? col : 0)) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[ks] = ok ? *reinterpret_cast<const u32x4*>(q_rot + off + 32 * ks) : u32x4{0, 0, 0, 0};
      ql[ks] = (ok && two_part) ? *reinterpret_cast<const u32x4*>(q_lo + off + 32 * ks)
                                : u32x4{0, 0, 0, 0};
    }
  };
  // K/V pages are read once per unit and never again in this step: non-temporal loads (the
  // streaming hint) raise the chip's read rate from ~6.2 to ~6.9 TB/s on 4 KB pages at random
  // addresses (measured with a plain read probe). A block id outside the pool reads block 0
  // (its page is masked in compute).
  auto page_base = [&](int b, int kh) {
    const bool in = b >= 0 && (long long)b < num_blocks;
    return ((size_t)(in ? b : 0) * Hkv + kh) * page_elems;
  };
  auto load_k = [&](const int* blk, int kh, Pair<D>& P) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t base = page_base(blk[h], kh);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        P.k[h][ks] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kpool + base + kpage_off(col, 4 * ks + lg)));
    }
  };
  auto load_v = [&](const int* blk, int kh, Pair<D>& P) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t base = page_base(blk[h], kh);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        P.v[h][mt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
            vpool + base + (size_t)(16 * mt + col) * HL_BLOCK_SIZE + 4 * lg));
    }
  };

  const bool carried = cy.item == item;
  const UnitRec rc = carried ? cy.rec : unit_rec(a.units, unit);
  const int pg0 = rc.pg0, nu = rc.nu, row = rc.row, kv_len = rc.kv_len;
  const int pg_end = pages_end(rc);
  const int32_t* __restrict__ trow = a.table + (size_t)rc.s * a.max_blocks;
  auto tbl = [&](int pa, int* blk) {
    const int p0 = min(pa, pg_end - 1), p1 = min(pa + 1, pg_end - 1);
    blk[0] = trow[p0];
    blk[1] = trow[p1];
  };

  u32x4 qf[D / 32], ql[D / 32];
  if (carried) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[ks] = cy.qf[ks];
      ql[ks] = cy.ql[ks];
    }
  } else {
    load_q(row, kvh, qf, ql);
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4{};
  float m_run = -1e30f, l_run = 0.f;

  // One page pair: the scores from P.k, after_k(), the softmax, P V from P.v, after_v().
  auto compute = [&](int pa, const int* blk, Pair<D>& P, auto after_k, auto after_v) {
    const int pb = pa + 1;
    const bool a_in = blk[0] >= 0 && (long long)blk[0] < num_blocks;
    const bool b_in = pb < pg_end && blk[1] >= 0 && (long long)blk[1] < num_blocks;
    f32x4 sa = f32x4{}, sb = f32x4{};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      sa = mfma16x16x32(P.k[0][ks], qf[ks], sa);
      sb = mfma16x16x32(P.k[1][ks], qf[ks], sb);
    }
    if (two_part) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        sa = mfma16x16x32(P.k[0][ks], ql[ks], sa);
        sb = mfma16x16x32(P.k[1][ks], ql[ks], sb);
      }
    }
    after_k();
    // lane (lg, col) holds tokens 4 lg + i of both pages for head col
    const int tok_a = pa * HL_BLOCK_SIZE + 4 * lg;
    const int tok_b = pb * HL_BLOCK_SIZE + 4 * lg;
    float tmax = -1e30f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = (a_in && tok_a + i < kv_len) ? sa[i] * scale_log2 : -INFINITY;
      sb[i] = (b_in && tok_b + i < kv_len) ? sb[i] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, fmaxf(sa[i], sb[i]));
    }
    tmax = wave_max_xor(tmax, 16);
    tmax = wave_max_xor(tmax, 32);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = fast_exp2(sa[i] - m_new);
      sb[i] = fast_exp2(sb[i] - m_new);
      psum += sa[i] + sb[i];
    }
    l_run = l_run * alpha + psum;
    // zero V of tokens past the end or of a page that is not used (weight 0, the slot may
    // hold anything)
    if (tok_b + 4 > kv_len || !a_in || !b_in) {
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t ma = ((a_in && tok_a + 2 * e < kv_len) ? 0xffffu : 0u) |
                              ((a_in && tok_a + 2 * e + 1 < kv_len) ? 0xffff0000u : 0u);
          const uint32_t mb = ((b_in && tok_b + 2 * e < kv_len) ? 0xffffu : 0u) |
                              ((b_in && tok_b + 2 * e + 1 < kv_len) ? 0xffff0000u : 0u);
          P.v[0][mt][e] &= ma;
          P.v[1][mt][e] &= mb;
        }
      }
    }
    // P^T operand: slots 0..3 = page a tokens 4 lg + i, slots 4..7 = page b tokens 4 lg + i
    const u32x4 pt = {pack_bf2(sa[0], sa[1]), pack_bf2(sa[2], sa[3]), pack_bf2(sb[0], sb[1]),
                      pack_bf2(sb[2], sb[3])};
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      o[mt] *= alpha;
      o[mt] = mfma16x16x32(u32x4{P.v[0][mt][0], P.v[0][mt][1], P.v[1][mt][0], P.v[1][mt][1]}, pt,
                           o[mt]);
    }
    after_v();
  };

  // The next item, as this wave learns it: the workgroup's claim, read once from LDS (thread 0
  // writes it when its claim returns; a wave that looks before that prefetches nothing).
  Carry<D> nc;
  nc.item = -1;
  nc.has_pair = false;
  bool polled = false;
  auto poll = [&]() {
    polled = true;
    const int nx = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(&L.tick, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (PREFETCH && nx >= 0 && nx < a.n_items) {
      nc.item = nx;
      nc.rec = unit_rec(a.units, nx / Hkv);
      unit_first_pair(a.units, nx / Hkv, wave, nc.blk);
    }
  };
  auto next_has_pair = [&]() {
    return nc.item >= 0 && nc.rec.pg0 + 2 * wave < pages_end(nc.rec);
  };

  // Software pipeline over this wave's page pairs (pairs p = pg0 + 2 wave + 8 i): while pair i
  // is computed, the K/V loads of pair i + 1 and the block-table reads of pair i + 2 are in
  // flight, so a wave never waits on a load it has just issued. The first pair's block ids come
  // with the record. With PREFETCH, in its second-to-last pair the wave reads the next item and
  // its record, and in its last pair it loads that item's first pair instead of a pair of this
  // item; the next item's query follows the last product.
  Pair<D> cur, nxt;
  const int first = pg0 + 2 * wave;
  if (first < pg_end) {
    int blk_cur[2], blk_nxt[2], blk_nn[2];
    if (carried && cy.has_pair) {
      blk_cur[0] = cy.blk[0];
      blk_cur[1] = cy.blk[1];
      cur = cy.first;
    } else {
      unit_first_pair(a.units, unit, wave, blk_cur);
      load_k(blk_cur, kvh, cur);
      load_v(blk_cur, kvh, cur);
    }
    tbl(first + 2 * kWaves, blk_nxt);
    for (int pa = first; pa < pg_end; pa += 2 * kWaves) {
      const bool last = pa + 2 * kWaves >= pg_end;
      if (!polled && pa + 4 * kWaves >= pg_end) poll();
      // table reads first: the load counter drains in issue order, so the next iteration can
      // wait for them without waiting for this iteration's K/V loads
      tbl(pa + 4 * kWaves, blk_nn);
      if (!last) {
        load_k(blk_nxt, kvh, nxt);
        load_v(blk_nxt, kvh, nxt);
      } else if (next_has_pair()) {
        load_k(nc.blk, nc.item % Hkv, nxt);
        load_v(nc.blk, nc.item % Hkv, nxt);
        nc.has_pair = true;
      }
      compute(pa, blk_cur, cur, [] {}, [] {});
      cur = nxt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        blk_cur[h] = blk_nxt[h];
        blk_nxt[h] = blk_nn[h];
      }
    }
  }
  if (!polled) {  // a wave with no pair in this item
    poll();
    if (next_has_pair()) {
      load_k(nc.blk, nc.item % Hkv, cur);
      load_v(nc.blk, nc.item % Hkv, cur);
      nc.has_pair = true;
    }
  }
  if (nc.item >= 0) {
    load_q(nc.rec.row, nc.item % Hkv, nc.qf, nc.ql);
    nc.first = cur;
  }

  // combine the waves' states; a lane's l covers its 8 tokens of each pair: sum over lg
  l_run = wave_sum_xor(l_run, 16);
  l_run = wave_sum_xor(l_run, 32);
  if (lg == 0) {
    sh_m[wave][col] = m_run;
    sh_l[wave][col] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sh_o[wave][16 * mt + 4 * lg + i][col] = o[mt][i];
  __syncthreads();

  // this unit's combined state for every head of the group
  if (nu == 1) {
    for (int e = tid; e < g * D; e += kThreads) {
      const int hh = e / D, d = e - hh * D;
      float mx = -1e30f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh_m[w][hh]);
      float acc = 0.f, lsum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = exp2f(sh_m[w][hh] - mx);
        acc += sh_o[w][d][hh] * sc;
        lsum += sh_l[w][hh] * sc;
      }
      attn_out[((size_t)row * Hq + kvh * g + hh) * D + d] = (hl_bf16)f2bf(acc / lsum);
    }
  } else {
    float* dst = part + ((size_t)rc.slot * Hkv + kvh) * g * (D + 2);
    for (int e = tid; e < g * D; e += kThreads) {
      const int hh = e / D, d = e - hh * D;
      float mx = -1e30f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh_m[w][hh]);
      float acc = 0.f, lsum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = exp2f(sh_m[w][hh] - mx);
        acc += sh_o[w][d][hh] * sc;
        lsum += sh_l[w][hh] * sc;
      }
      dst[hh * (D + 2) + d] = acc;
      if (d == 0) {
        dst[hh * (D + 2) + D] = mx;
        dst[hh * (D + 2) + D + 1] = lsum;
      }
    }
  }
  cy = nc;
  return rc.slot * Hkv + kvh;
}

}  // namespace decode
}  // namespace hl
