// One split-KV decode work unit (a run of pages of one decode sequence, one KV head), shared by
// the standalone decode-attention kernel and the fused hybrid-attention kernel. The method and the
// design are described in attention_decode.hip.
#pragma once
#include "common.h"

namespace hl {
namespace decode {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

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
  const int32_t* units;     // [n][3]: (sequence, first page, decode index)
  const int32_t* dec_seqs;  // [n][3]: (sequence, first unit, unit count)
  int split_pages;
  int Hq, Hkv;
  float scale_log2;
  float* part;
  hl_bf16* attn_out;
};

// LDS of one work unit: the waves' (o, m, l) states before they are combined.
template <int D>
struct DecodeLds {
  float o[kWaves][D][16];
  float m[kWaves][16];
  float l[kWaves][16];
};

// Work unit `unit`, KV head kvh. Every thread of a kThreads-thread workgroup calls it. Consecutive
// units of one workgroup must be separated by a barrier (the LDS is reused).
template <int D>
HL_DEV void decode_unit(const DecodeArgs& a, int unit, int kvh, DecodeLds<D>& L) {
  const int32_t* __restrict__ q_start = a.q_start;
  const int32_t* __restrict__ num_cached = a.num_cached;
  const hl_bf16* __restrict__ q_rot = a.q_rot;
  const hl_bf16* __restrict__ q_lo = a.q_lo;
  const hl_bf16* __restrict__ kpool = a.kpool;
  const hl_bf16* __restrict__ vpool = a.vpool;
  const long long num_blocks = a.num_blocks;
  const int32_t* __restrict__ table = a.table;
  const int max_blocks = a.max_blocks, split_pages = a.split_pages, Hq = a.Hq, Hkv = a.Hkv;
  const float scale_log2 = a.scale_log2;
  const int32_t* __restrict__ dec_seqs = a.dec_seqs;
  float* __restrict__ part = a.part;
  hl_bf16* __restrict__ attn_out = a.attn_out;
  auto& sh_o = L.o;
  auto& sh_m = L.m;
  auto& sh_l = L.l;
  const int s = a.units[3 * unit], pg0 = a.units[3 * unit + 1], di = a.units[3 * unit + 2];
  const int u0 = dec_seqs[3 * di + 1], nu = dec_seqs[3 * di + 2];
  const int row = q_start[s];
  const int kv_len = num_cached[s] + 1;
  const int npages = (kv_len + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
  const int pg_end = min(pg0 + split_pages, npages);
  const int g = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4;   // lane group 0..3
  const int col = lane & 15;  // S^T / O^T column = query head within the group
  const int32_t* trow = table + (size_t)s * max_blocks;
  const size_t page_elems = (size_t)HL_BLOCK_SIZE * D;

  // Q^T operand: lane (lg, col) holds head col, d = 32 ks + 8 lg .. +7
  u32x4 qf[D / 32], ql[D / 32];
  const bool two_part = q_lo != nullptr;
  {
    const bool ok = col < g;
    const size_t off = ((size_t)row * Hq + kvh * g + (ok ? col : 0)) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[ks] = ok ? *reinterpret_cast<const u32x4*>(q_rot + off + 32 * ks) : u32x4{0, 0, 0, 0};
      ql[ks] = (ok && two_part) ? *reinterpret_cast<const u32x4*>(q_lo + off + 32 * ks)
                                : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4{};
  float m_run = -1e30f, l_run = 0.f;

  // Software pipeline over this wave's page pairs (pairs p = pg0 + 2 wave + 8 i): while pair i
  // is computed, the K/V loads of pair i + 1 and the block-table reads of pair i + 2 are in
  // flight, so a wave never waits on a load it has just issued. Past the last pair the loads
  // repeat the unit's last page (in bounds) and their results are not used.
  struct Pair {
    u32x4 k[2][D / 32];
    u32x2 v[2][D / 16];
  };
  auto tbl = [&](int pa, int* blk) {
    const int p0 = min(pa, pg_end - 1), p1 = min(pa + 1, pg_end - 1);
    blk[0] = trow[p0];
    blk[1] = trow[p1];
  };
  // K/V pages are read once per unit and never again in this step: non-temporal loads (the
  // streaming hint) raise the chip's read rate from ~6.2 to ~6.9 TB/s on 4 KB pages at random
  // addresses (measured with a plain read probe)
  auto load = [&](const int* blk, Pair& P) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool in = blk[h] >= 0 && (long long)blk[h] < num_blocks;
      const size_t base = ((size_t)(in ? blk[h] : 0) * Hkv + kvh) * page_elems;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        P.k[h][ks] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kpool + base + kpage_off(col, 4 * ks + lg)));
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        P.v[h][mt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
            vpool + base + (size_t)(16 * mt + col) * HL_BLOCK_SIZE + 4 * lg));
    }
  };
  auto compute = [&](int pa, const int* blk, Pair& P) {
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
  };

  const int first = pg0 + 2 * wave;
  if (first < pg_end) {
    int blk_cur[2], blk_nxt[2], blk_nn[2];
    Pair cur, nxt;
    tbl(first, blk_cur);
    load(blk_cur, cur);
    tbl(first + 2 * kWaves, blk_nxt);
    for (int pa = first; pa < pg_end; pa += 2 * kWaves) {
      // table reads first: the load counter drains in issue order, so the next iteration can
      // wait for them without waiting for this iteration's K/V loads
      tbl(pa + 4 * kWaves, blk_nn);
      load(blk_nxt, nxt);
      compute(pa, blk_cur, cur);
      cur = nxt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        blk_cur[h] = blk_nxt[h];
        blk_nxt[h] = blk_nn[h];
      }
    }
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
    return;
  }
  float* dst = part + ((size_t)unit * Hkv + kvh) * g * (D + 2);
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

}  // namespace decode
}  // namespace hl
