// Device-side work lists of one step, derived from the batch descriptor's device arrays.
//
// Each sequence is either a decode (one new token) or a prompt chunk (several new tokens at
// offset num_cached), the two kinds a chunked-prefill iteration mixes ("Chunked prefill
// (stall-free batching), explained", "How it works, step by step"). One workgroup classifies
// the sequences and scans their work counts:
//   decode unit  = (sequence, first page, decode index) covering `split_pages` KV pages;
//   decode entry = (sequence, first unit, unit count) for the split merge;
//   prefill entry = (sequence, first query row, key-tile range, partial slot): a tile of
//                  `kPrefillQTile` query rows, or one part of it when its causal key range is
//                  longer than `pre_split` key tiles (a few long items would otherwise leave most
//                  compute units idle: short chunks after a long cached prefix, the last tiles of
//                  a causal chunk); tiles are emitted last tile first, so the longest key ranges
//                  are dispatched first;
//   prefill merge = (sequence, first query row, first slot, part count) for each split tile.
// The host computes the same counts from its mirrors to size the grids, so nothing is read back.
#pragma once
#include "common.h"

namespace hl {
namespace plan {

// Exclusive scan of N counts per thread across the workgroup, all N at once: a shuffle scan
// inside each wave, then the wave totals through LDS (two barriers for all N).
template <int NT, int N>
HL_DEV void block_exclusive_scan(const int (&v)[N], int (&off)[N], int (&total)[N],
                                 int (*wt)[NT / 64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = v[i];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc[i], d, 64);
      if (lane >= d) inc[i] += o;
    }
    if (lane == 63) wt[i][wave] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int before = 0, all = 0;
    for (int w = 0; w < NT / 64; ++w) {
      before += (w < wave) ? wt[i][w] : 0;
      all += wt[i][w];
    }
    off[i] = before + inc[i] - v[i];
    total[i] = all;
  }
  __syncthreads();  // wt may be rewritten by the next call
}

// The work lists of the batch, built by one workgroup of NT threads (every thread calls it);
// `wt` is NT / 64 ints x 5 of LDS.
template <int NT>
HL_DEV void build(const int32_t* __restrict__ q_start, const int32_t* __restrict__ num_cached,
                  int num_seqs, const int32_t* __restrict__ table, int max_blocks,
                  const hl::Plan& p, int (*wt)[NT / 64]) {
  constexpr int QT = hl::kPrefillQTile;
  if (threadIdx.x < hl::kPlanCounters) p.counters[threadIdx.x * hl::kCounterStride] = 0;
  int base_u = 0, base_d = 0, base_e = 0, base_p = 0, base_m = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += NT) {
    const int s = s0 + threadIdx.x;
    int units = 0, is_dec = 0, ents = 0, slots = 0, merges = 0, qlen = 0, c = 0;
    if (s < num_seqs) {
      qlen = q_start[s + 1] - q_start[s];
      c = num_cached[s];
      const int kv = c + qlen;
      if (qlen == 1) {
        const int pages = (kv + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
        units = (pages + p.split_pages - 1) / p.split_pages;
        is_dec = 1;
      } else if (qlen > 1) {
        for (int r0 = 0; r0 < qlen; r0 += QT) {
          const int parts = hl::prefill_parts(hl::prefill_key_tiles(c, r0, min(QT, qlen - r0)),
                                              p.pre_split);
          ents += parts;
          if (parts > 1) {
            slots += parts;
            merges += 1;
          }
        }
      }
    }
    const int cnt[5] = {units, is_dec, ents, slots, merges};
    int off[5], tot[5];
    block_exclusive_scan<NT, 5>(cnt, off, tot, wt);
    const int off_u = base_u + off[0], off_d = base_d + off[1], off_e = base_e + off[2],
              off_p = base_p + off[3], off_m = base_m + off[4];
    if (is_dec) {
      const int row = q_start[s];
      const int pages = (c + qlen + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
      const int32_t* trow = table + (size_t)s * max_blocks;
      for (int u = 0; u < units; ++u) {
        int32_t* r = p.dec_units + (size_t)hl::kDecUnitInts * (off_u + u);
        const int pg0 = u * p.split_pages, last = min(pg0 + p.split_pages, pages) - 1;
        r[0] = s;
        r[1] = pg0;
        r[2] = off_d;
        r[3] = units;
        r[4] = row;
        r[5] = c + qlen;
        r[6] = 0;
        r[7] = 0;
        for (int j = 0; j < 8; ++j) r[8 + j] = trow[min(pg0 + j, last)];
      }
      p.dec_seqs[3 * off_d] = s;
      p.dec_seqs[3 * off_d + 1] = off_u;
      p.dec_seqs[3 * off_d + 2] = units;
    }
    if (ents > 0) {
      int e = off_e, slot = off_p, m = off_m;
      for (int r0 = ((qlen - 1) / QT) * QT; r0 >= 0; r0 -= QT) {
        const int nkt = hl::prefill_key_tiles(c, r0, min(QT, qlen - r0));
        const int parts = hl::prefill_parts(nkt, p.pre_split);
        for (int j = 0; j < parts; ++j, ++e) {
          int32_t* t = p.pre_tiles + (size_t)hl::kPreEntry * e;
          t[0] = s;
          t[1] = r0;
          t[2] = (int)((long long)j * nkt / parts);  // near-equal parts
          t[3] = (int)((long long)(j + 1) * nkt / parts);
          t[4] = parts > 1 ? slot + j : -1;
        }
        if (parts > 1) {
          p.pre_merge[4 * m] = s;
          p.pre_merge[4 * m + 1] = r0;
          p.pre_merge[4 * m + 2] = slot;
          p.pre_merge[4 * m + 3] = parts;
          slot += parts;
          ++m;
        }
      }
    }
    base_u += tot[0];
    base_d += tot[1];
    base_e += tot[2];
    base_p += tot[3];
    base_m += tot[4];
  }
}

}  // namespace plan
}  // namespace hl
