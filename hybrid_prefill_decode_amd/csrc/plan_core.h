// Device-side work lists of one step, derived from the batch descriptor's device arrays.
//
// Each sequence is either a decode (one new token) or a prompt chunk (several new tokens at
// offset num_cached), the two kinds a chunked-prefill iteration mixes ("Chunked prefill
// (stall-free batching), explained", "How it works, step by step"). A few workgroups (build())
// classify the sequences, scan their work counts and write:
//   decode unit  = (sequence, first page, decode index) covering `split_pages` KV pages, stored
//                  in sequence order or (dec_lpt) in dispatch order (largest first, dealt
//                  round-robin to 8 runs: dec_position), with its index in sequence order as
//                  its partial slot;
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

// Inclusive sum over the lanes of a wave, lane 0 first: four shifts within each row of 16 lanes,
// then row 15's sum into rows 1 and 3 and row 31's into rows 2 and 3 (DPP row_shr and row_bcast
// on the VALU; a lane with no source adds 0).
HL_DEV int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive scan of N counts per thread across the workgroup, all N at once: a scan inside each
// wave, then a scan of the wave totals passed through LDS (two barriers for all N).
template <int NT, int N>
HL_DEV void block_exclusive_scan(const int (&v)[N], int (&off)[N], int (&total)[N],
                                 int (*wt)[NT / 64]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = wave_incl_scan(v[i]);
    if (lane == 63) wt[i][wave] = inc[i];
  }
  __syncthreads();
  // the wave totals scanned across the lanes of every wave alike: lane w holds wave w's total
  constexpr int W = NT / 64;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int x = wave_incl_scan(lane < W ? wt[i][lane] : 0);
    const int before = wave > 0 ? __builtin_amdgcn_readlane(x, wave - 1) : 0;
    total[i] = __builtin_amdgcn_readlane(x, W - 1);
    off[i] = before + inc[i] - v[i];
  }
  __syncthreads();  // wt may be rewritten by the next call
}

// LDS of build() for a workgroup of NT threads.
template <int NT>
struct Shared {
  int wt[4 + hl::kDecBuckets / 2][NT / 64];  // wave totals of the scans
  int off_u[NT + 1];    // per sequence of the current block: first decode unit (block-relative)
  int off_t[NT + 1];    // first prefill query tile (block-relative)
  int row[NT];          // first token row of the sequence
  int cached[NT];       // cached prefix length
  int kv[NT];           // KV length after the step
  int dseq[NT];         // decode index (position in dec_seqs)
  int full_rank[NT];    // dispatch rank of the sequence's first full unit
  int last_rank[NT];    // dispatch rank of its shorter last unit, or -1 if all units are full
  int e_off[NT + 1];    // per prefill query tile of the current pass: first entry (pass-relative)
  int e_seq[NT];        // its sequence
  int e_r0[NT];         // its first query row
  int e_nkt[NT];        // its key tiles
  int e_slot[NT];       // its first partial slot (or -1 when unsplit)
};

// Largest i < n with off[i] <= k (off non-decreasing, off[0] = 0 <= k): the sequence whose run
// of items holds item k. Sequences with no items share the next one's offset and are skipped.
HL_DEV int owner(const int* off, int n, int k) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= k) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The work lists of the batch, built by nwg workgroups of NT threads (every thread of workgroup
// wg calls it). Sequences are taken NT at a time: each thread classifies one and the workgroup
// scans the counts; then the decode units and the prefill query tiles of those sequences are
// dealt over the threads of all nwg workgroups (a thread finds its item's sequence by binary
// search over the scanned offsets), so no thread writes a long sequence's records alone and the
// scattered table reads and record stores spread over nwg compute units. Every workgroup runs the
// same scans (cheap) and writes only its share of the records. A thread gathers the block ids of
// up to kBatch units before it stores any record: loads queued behind stores would wait for them.
template <int NT>
HL_DEV void build(const int32_t* __restrict__ q_start, const int32_t* __restrict__ num_cached,
                  int num_seqs, const int32_t* __restrict__ table, int max_blocks,
                  const hl::Plan& p, Shared<NT>& sh, int wg, int nwg) {
  constexpr int QT = hl::kPrefillQTile;
  constexpr int kBatch = NT >= 1024 ? 2 : 4;  // within the 128 registers of 1024 threads
  if (wg == 0 && threadIdx.x < hl::kPlanCounters) p.counters[threadIdx.x * hl::kCounterStride] = 0;
  int base_u = 0, base_d = 0, base_e = 0, base_p = 0, base_m = 0, base_f = 0;
  int base_b[hl::kDecBuckets] = {};
  for (int s0 = 0; s0 < num_seqs; s0 += NT) {
    const int t = threadIdx.x, s = s0 + t;
    int units = 0, is_dec = 0, tiles = 0, row = 0, c = 0, qlen = 0, full = 0, bucket = -1;
    if (s < num_seqs) {
      row = q_start[s];
      qlen = q_start[s + 1] - row;
      c = num_cached[s];
      if (qlen == 1) {
        const int pages = (c + 1 + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
        units = (pages + p.split_pages - 1) / p.split_pages;
        is_dec = 1;
        const int rem = pages % p.split_pages;
        full = units - (rem ? 1 : 0);
        if (rem) bucket = hl::dec_bucket(rem, p.split_pages);
      } else if (qlen > 1) {
        tiles = (qlen + QT - 1) / QT;
      }
    }
    // the size classes two to an int (16 bits each: at most NT per round)
    int cnt[4 + hl::kDecBuckets / 2] = {units, is_dec, tiles, full};
#pragma unroll
    for (int j = 0; j < hl::kDecBuckets / 2; ++j)
      cnt[4 + j] = bucket == 2 * j ? 1 : (bucket == 2 * j + 1 ? 1 << 16 : 0);
    int off[4 + hl::kDecBuckets / 2], tot[4 + hl::kDecBuckets / 2];
    block_exclusive_scan<NT, 4 + hl::kDecBuckets / 2>(cnt, off, tot, sh.wt);
    sh.off_u[t] = off[0];
    sh.off_t[t] = off[2];
    sh.row[t] = row;
    sh.cached[t] = c;
    sh.kv[t] = c + qlen;
    sh.dseq[t] = base_d + off[1];
    sh.full_rank[t] = base_f + off[3];
    sh.last_rank[t] = -1;
#pragma unroll
    for (int k = 0; k < hl::kDecBuckets; ++k)
      if (bucket == k)
        sh.last_rank[t] = p.dec_rank_base[k] + base_b[k] + ((off[4 + k / 2] >> (16 * (k & 1))) & 0xffff);
    if (is_dec && s % nwg == wg) {
      p.dec_seqs[3 * (base_d + off[1])] = s;
      p.dec_seqs[3 * (base_d + off[1]) + 1] = base_u + off[0];
      p.dec_seqs[3 * (base_d + off[1]) + 2] = units;
    }
    if (t == 0) {
      sh.off_u[NT] = tot[0];
      sh.off_t[NT] = tot[2];
    }
    __syncthreads();

    // decode units: 64-byte records, kBatch per thread per round
    const int ustep = nwg * NT;  // unit k belongs to workgroup (k / NT) % nwg
    for (int k0 = wg * NT + t; k0 < tot[0]; k0 += kBatch * ustep) {
      int ids[kBatch][8], own[kBatch], pg[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int k = k0 + b * ustep;
        if (k < tot[0]) {
          const int i = owner(sh.off_u, NT, k);
          const int pages = (sh.kv[i] + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
          const int pg0 = (k - sh.off_u[i]) * p.split_pages;
          const int last = min(pg0 + p.split_pages, pages) - 1;
          const int32_t* trow = table + (size_t)(s0 + i) * max_blocks;
#pragma unroll
          for (int j = 0; j < 8; ++j) ids[b][j] = trow[min(pg0 + j, last)];
          own[b] = i;
          pg[b] = pg0;
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int k = k0 + b * ustep, i = own[b];
        if (k < tot[0]) {
          const int nu = sh.off_u[i + 1] - sh.off_u[i], u = k - sh.off_u[i];
          const int last = sh.last_rank[i];
          const int rank = (last >= 0 && u == nu - 1) ? last : sh.full_rank[i] + u;
          const int pos = p.dec_lpt ? hl::dec_position(rank, p.n_dec_units) : base_u + k;
          int4* r = reinterpret_cast<int4*>(p.dec_units + (size_t)hl::kDecUnitInts * pos);
          r[0] = make_int4(s0 + i, pg[b], sh.dseq[i], nu);
          r[1] = make_int4(sh.row[i], sh.kv[i], base_u + k, 0);
          r[2] = make_int4(ids[b][0], ids[b][1], ids[b][2], ids[b][3]);
          r[3] = make_int4(ids[b][4], ids[b][5], ids[b][6], ids[b][7]);
        }
      }
    }

    // prefill query tiles, each sequence's last tile first (the longest key ranges are
    // dispatched first); a tile whose key range exceeds pre_split key tiles becomes near-equal
    // parts with partial slots and one merge record
    for (int k0 = 0; k0 < tot[2]; k0 += NT) {
      const int k = k0 + t;
      int i = 0, r0 = 0, nkt = 0, parts = 0;
      if (k < tot[2]) {
        i = owner(sh.off_t, NT, k);
        const int ql = sh.kv[i] - sh.cached[i];
        r0 = ((ql - 1) / QT - (k - sh.off_t[i])) * QT;
        nkt = hl::prefill_key_tiles(sh.cached[i], r0, min(QT, ql - r0));
        parts = hl::prefill_parts(nkt, p.pre_split);
      }
      const int pc[3] = {parts, parts > 1 ? parts : 0, parts > 1 ? 1 : 0};
      int po[3], pt[3];
      block_exclusive_scan<NT, 3>(pc, po, pt, sh.wt);
      sh.e_off[t] = po[0];
      sh.e_seq[t] = s0 + i;
      sh.e_r0[t] = r0;
      sh.e_nkt[t] = nkt;
      sh.e_slot[t] = parts > 1 ? base_p + po[1] : -1;
      if (t == 0) sh.e_off[NT] = pt[0];
      if (parts > 1 && k % nwg == wg) {
        int32_t* m = p.pre_merge + 4 * (size_t)(base_m + po[2]);
        m[0] = s0 + i;
        m[1] = r0;
        m[2] = base_p + po[1];
        m[3] = parts;
      }
      __syncthreads();
      // the entries of the pass, one per thread: part j of n covers key tiles
      // [j * nkt / n, (j + 1) * nkt / n) (near-equal parts)
      for (int e = wg * NT + t; e < pt[0]; e += nwg * NT) {
        const int tl = owner(sh.e_off, NT, e);
        const int j = e - sh.e_off[tl], n = sh.e_off[tl + 1] - sh.e_off[tl];
        const int nk = sh.e_nkt[tl], slot = sh.e_slot[tl];
        int first, end;
        if (nk <= 46340) {  // (j + 1) * nk stays below 2^31
          first = (int)((unsigned)(j * nk) / (unsigned)n);
          end = (int)((unsigned)((j + 1) * nk) / (unsigned)n);
        } else {
          first = (int)((long long)j * nk / n);
          end = (int)((long long)(j + 1) * nk / n);
        }
        int32_t* r = p.pre_tiles + (size_t)hl::kPreEntry * (base_e + e);
        r[0] = sh.e_seq[tl];
        r[1] = sh.e_r0[tl];
        r[2] = first;
        r[3] = end;
        r[4] = slot >= 0 ? slot + j : -1;
      }
      base_e += pt[0];
      base_p += pt[1];
      base_m += pt[2];
    }
    base_u += tot[0];
    base_d += tot[1];
    base_f += tot[3];
#pragma unroll
    for (int k = 0; k < hl::kDecBuckets; ++k) base_b[k] += (tot[4 + k / 2] >> (16 * (k & 1))) & 0xffff;
  }
}

}  // namespace plan
}  // namespace hl
