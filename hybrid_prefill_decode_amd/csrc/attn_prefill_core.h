// One ragged causal prefill work item (128 query rows of one sequence, one query head, a range of
// its key tiles), shared by the standalone prefill-attention kernel and the fused hybrid-attention
// kernel. The method and the design are described in attention_prefill.hip.
#pragma once
#include <type_traits>

#include "common.h"

namespace hl {
namespace prefill {


constexpr int kThreads = 256;
constexpr int kKeys = kPrefillKeyTile;  // keys per step = 4 pages
static_assert(kKeys == 64 && kPrefillQTile == 128, "the item's tiling");

template <int D>
struct PrefillSmem {
  static constexpr int kKBytes = kKeys * D * 2;     // K tile [64][D]
  static constexpr int kVBytes = 4 * D * 32;        // V^T tile [4 pages][D][16]
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
  static constexpr int kChunks = kKBytes / 16;      // 16-byte chunks of K (same count for V)
  static constexpr int kPer = kChunks / kThreads;   // per thread: 4 (D = 128) or 2 (D = 64)
  static constexpr int kChunksPerPage = kChunks / 4;
};

// K tile rows of D*2 bytes; the 16-byte chunk c of row r is XOR-swizzled so that the 16 lanes of
// one read group (rows r..r+15, same chunk) hit distinct banks.
template <int D>
HL_DEV int k_off(int r, int c) {
  if (D == 128) return r * 256 + ((c ^ (r & 15)) << 4);
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
// V^T tile: dim row d of page pg holds its 16 tokens in quad order (0, 2, 1, 3), so that the
// 16 bytes the P V product needs in lane half h (tokens 4h..4h+3 and 8+4h..8+4h+3) are contiguous;
// the two 16-byte halves of rows d and d + 8 are swapped so 16 consecutive rows hit distinct banks.
template <int D>
HL_DEV int v_off(int pg, int d, int half) {
  return pg * D * 32 + d * 32 + ((half ^ ((d >> 3) & 1)) << 4);
}

struct PrefillArgs {
  const int32_t* q_start;
  const int32_t* num_cached;
  const hl_bf16* q_rot;
  const hl_bf16* kpool;
  const hl_bf16* vpool;
  long long num_blocks;
  const int32_t* table;
  int max_blocks;
  const int32_t* tiles;  // [n][kPreEntry]: (sequence, first query row, key tiles [kt0, kt1),
                         // partial slot or -1)
  int Hq, Hkv;
  float scale_log2;
  hl_bf16* attn_out;
  float* part_o;         // [slot][Hq][128][D]: unnormalised o of a part
  float2* part_ml;       // [slot][Hq][128]: (m, l) of a part, m in the exp2 domain
  uint64_t* trace;       // optional: work-item trace records (Plan::trace), prefill items first
};

// Work item (entry, query head h): the entry's query rows against its key tiles [kt0, kt1). An
// entry that covers the tile's whole key range writes the normalised rows; a part of a split tile
// writes its unnormalised o and its (m, l) to slot `slot`, and a merge pass combines the parts.
// Every thread of a kThreads-thread workgroup calls it; `smem` holds PrefillSmem<D>::kTotal
// bytes. Consecutive items of one workgroup must be separated by a barrier (the LDS stages are
// reused).
template <int D>
HL_DEV void prefill_item(const PrefillArgs& a, int tile, int h, uint8_t* smem) {
  using SM = PrefillSmem<D>;
  const int32_t* __restrict__ q_start = a.q_start;
  const int32_t* __restrict__ num_cached = a.num_cached;
  const hl_bf16* __restrict__ q_rot = a.q_rot;
  const hl_bf16* __restrict__ kpool = a.kpool;
  const hl_bf16* __restrict__ vpool = a.vpool;
  const long long num_blocks = a.num_blocks;
  const int32_t* __restrict__ table = a.table;
  const int max_blocks = a.max_blocks, Hq = a.Hq, Hkv = a.Hkv;
  const float scale_log2 = a.scale_log2;
  hl_bf16* __restrict__ attn_out = a.attn_out;
  const int g = Hq / Hkv;
  const int32_t* ent = a.tiles + (size_t)kPreEntry * tile;
  const int s = ent[0], r0 = ent[1], kt0 = ent[2], kt1 = ent[3], slot = ent[4];
  const int qs = q_start[s], n = q_start[s + 1] - qs, c = num_cached[s];
  const int kvh = h / g;
  const int kv_len = c + n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl32 = lane >> 5;
  const int tile_rows = min(128, n - r0);
  const int nkt = prefill_key_tiles(c, r0, tile_rows);  // key tiles of the whole tile
  const int wr0 = r0 + 32 * wave;
  const int my_row = wr0 + (lane & 31);
  const bool row_ok = my_row < n;
  const int qpos = row_ok ? c + my_row : -1;
  const int32_t* trow = table + (size_t)s * max_blocks;
  const size_t page_elems = (size_t)HL_BLOCK_SIZE * D;

  // Q^T operand: slot j of lane-half hl32 at k-step ks holds d = 16 ks + 8 hl32 + j
  u32x4 qf[D / 16];
  {
    const hl_bf16* qp = q_rot + ((size_t)(qs + (row_ok ? my_row : 0)) * Hq + h) * D + 8 * hl32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0, 0, 0, 0};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  // Per-thread slice of a key tile: 16-byte chunk q = tid + kThreads * i lies in page
  // pg = q / kChunksPerPage at element offset w * 8, w = q % kChunksPerPage. Consecutive i step
  // the page by kThreads / kChunksPerPage and every LDS destination by 4096 bytes.
  constexpr int kPagesPerI = kThreads / SM::kChunksPerPage;
  const int pg0 = tid / SM::kChunksPerPage, w = tid % SM::kChunksPerPage;
  // K: chunk w of a chunk-major page is token w % 16, chunk w / 16
  const int k_dst = k_off<D>(pg0 * 16 + w % 16, w / 16);
  // V^T: this thread moves chunk wv of the page, w with bits 3 and 4 swapped, so that each
  // 16 lanes store rows {0..3, 8..11} (+ 4 or 16 multiples) and their 8-byte pieces fall in
  // distinct banks. Chunk wv is dim row wv / 2, token quads 2 (wv & 1) and 2 (wv & 1) + 1, which
  // sit at quad positions (wv & 1) and 2 + (wv & 1).
  const int wv = (w & ~24) | ((w & 8) << 1) | ((w & 16) >> 1);
  const int v_dst0 = v_off<D>(pg0, wv >> 1, 0) + 8 * (wv & 1);
  const int v_dst1 = v_off<D>(pg0, wv >> 1, 1) + 8 * (wv & 1);
  static_assert(kPagesPerI * 16 * D * 2 == 4096 && kPagesPerI * D * 32 == 4096, "tile slice");
  // byte addresses: page base + this thread's chunk; a block adds blk * block_bytes
  const uint32_t block_bytes = (uint32_t)(Hkv * page_elems * 2);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kpool) + (size_t)kvh * page_elems * 2 + 16 * w;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vpool) + (size_t)kvh * page_elems * 2 + 16 * wv;
  const uint32_t nb = (uint32_t)min(num_blocks, (long long)INT32_MAX);

  u32x4 rk[SM::kPer], rv[SM::kPer];
  int blk[SM::kPer];
  const int npages = (kv_len + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE;
  // Three-stage software pipeline over key tiles: step kt stores tile kt + 1 to LDS, issues the
  // K/V loads of tile kt + 2 and the block-table reads of tile kt + 3, each from data that
  // arrived during the previous step, so no step waits on a load it issued itself. The stores
  // and loads go in the second half of the step, one slice per page of the P V product, after
  // that page's V fragment reads: the score products then wait only for their own K fragment
  // reads (the LDS counter drains in issue order, so stores issued before them would hold the
  // first product back), and the stores overlap the exponentials. Loads are unconditional: a
  // page past the sequence repeats the last page, whose surplus rows are masked (K by the score
  // mask, V by zeroing in sstore); invalid table entries read block 0.
  auto tload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < SM::kPer; ++i)
      blk[i] = trow[min(4 * kt + pg0 + kPagesPerI * i, npages - 1)];
  };
  auto gload1 = [&](int i) {
    const uint32_t b = ((uint32_t)blk[i] < nb) ? (uint32_t)blk[i] : 0u;
    const size_t off = (size_t)b * block_bytes;
    rk[i] = *reinterpret_cast<const u32x4*>(kbase + off);
    rv[i] = *reinterpret_cast<const u32x4*>(vbase + off);
  };
  auto gload = [&]() {
#pragma unroll
    for (int i = 0; i < SM::kPer; ++i) gload1(i);
  };
  // ZERO: V rows past the sequence end are zeroed when stored (their weight is 0, the slot may
  // hold anything, and 0 * NaN would poison the product); only the last tile has such rows.
  // Slice i of the thread's part of the tile.
  auto sstore1 = [&](int buf, int kt, int i, auto zero) {
    uint8_t* kb = smem + buf * SM::kStage;
    uint8_t* vb = kb + SM::kKBytes;
    {
      u32x4 vv = rv[i];
      if constexpr (decltype(zero)::value) {
        const int tok0 = (4 * kt + pg0 + kPagesPerI * i) * HL_BLOCK_SIZE + 8 * (wv & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo_ok = (tok0 + 2 * e < kv_len) ? 0x0000ffffu : 0u;
          const uint32_t hi_ok = (tok0 + 2 * e + 1 < kv_len) ? 0xffff0000u : 0u;
          vv[e] &= (lo_ok | hi_ok);
        }
      }
      *reinterpret_cast<u32x4*>(kb + k_dst + 4096 * i) = rk[i];
      *reinterpret_cast<u32x2*>(vb + v_dst0 + 4096 * i) = u32x2{vv[0], vv[1]};
      *reinterpret_cast<u32x2*>(vb + v_dst1 + 4096 * i) = u32x2{vv[2], vv[3]};
    }
  };
  auto sstore = [&](int buf, int kt, auto zero) {
#pragma unroll
    for (int i = 0; i < SM::kPer; ++i) sstore1(buf, kt, i, zero);
  };
  const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)

  // One key tile. MASKED: keys past a query's position are masked and the stored tile's V rows
  // past the sequence end are zeroed; both are needed only on the last few tiles of a query tile.
  auto step = [&](int kt, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int buf = kt & 1;
    const uint8_t* kb = smem + buf * SM::kStage;
    // S^T for the two 32-key halves of the tile; half hb holds keys
    // 32 hb + 8 (i / 4) + 4 hl32 + (i & 3) of query lane & 31
    f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 ka =
            *reinterpret_cast<const u32x4*>(kb + k_off<D>(32 * hb + (lane & 31), 2 * ks + hl32));
        st[hb] = mfma32x32x16(ka, qf[ks], st[hb]);
      }
    if constexpr (kMasked) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt * kKeys + 32 * hb + 8 * (i >> 2) + 4 * hl32 + (i & 3);
          st[hb][i] = (key <= qpos) ? st[hb][i] : -INFINITY;
        }
    }
    // V fragments of page 0 (each page's are read one page ahead of its products)
    const uint8_t* vb = kb + SM::kKBytes;
    u32x4 va[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
      va[mt] = *reinterpret_cast<const u32x4*>(vb + v_off<D>(0, 32 * mt + (lane & 31), hl32));
    // Softmax in the exp2 domain with the scale folded in: the max is taken on raw scores and
    // p = 2^(s * scale_log2 - m) costs one FMA and one exp2.
    float tmax = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(st[hb][i], st[hb][i + 1]));
    // K fragment reads running three ahead of the score products
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS read
#pragma unroll
    for (int q = 0; q < D / 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (q < D / 8 - 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    tmax = wave_max_xor(tmax, 32) * scale_log2;
    // Lazy rescaling: the reference m_run moves only when a tile max exceeds it by more than 8,
    // so every p stays <= 2^8 (far inside fp32 / bf16 range) and most tiles skip the rescale of
    // o and l; o / l does not depend on the reference. The branch is taken wave-wide (a lane
    // that did not need it rescales by its own alpha <= 1, which is equally valid).
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + 8.f)) {
      const float m_new = fmaxf(tmax, m_run);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
    }
    // Page by page: the weights of page t (P^T operand: half t / 2, regs 8 (t % 2) .. +7), their
    // sum (taken from the same bf16 weights that multiply V, by a packed dot product with
    // (1, 1)), then the page's D / 32 products, so the exponentials of page t + 1 overlap the
    // matrix cores working on page t.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(st[t >> 1][8 * (t & 1) + 2 * e], scale_log2, -m_run));
        const float p1 = fast_exp2(fmaf(st[t >> 1][8 * (t & 1) + 2 * e + 1], scale_log2, -m_run));
        pb[e] = pack_bf2(p0, p1);
        l_run = dot2_bf16(pb[e], ones, l_run);
      }
      u32x4 vn[D / 32];
      if (t < 3) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
          vn[mt] =
              *reinterpret_cast<const u32x4*>(vb + v_off<D>(t + 1, 32 * mt + (lane & 31), hl32));
      }
      // slice t of the next tile into the other buffer (last read one step ago, before the
      // barrier), then the loads of the tile after it into the freed registers (past the end
      // they repeat the last tile, unused)
      if (t < SM::kPer) {
        sstore1(buf ^ 1, min(kt + 1, kt1 - 1), t, masked);
        gload1(t);
      }
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) o[mt] = mfma32x32x16(va[mt], pb, o[mt]);
      if (t < 3) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) va[mt] = vn[mt];
      }
    }
    tload(min(kt + 3, kt1 - 1));
    __syncthreads();
  };

  tload(kt0);
  gload();
  tload(min(kt0 + 1, kt1 - 1));
  sstore(kt0 & 1, kt0, std::true_type{});
  gload();
  tload(min(kt0 + 2, kt1 - 1));
  __syncthreads();
  // Tiles wholly at or below the tile's first query position need neither the mask nor V
  // zeroing (only the last of the tile's key tiles holds rows past the sequence end); the step
  // before the first tile that needs them already stores it, so runs masked.
  const int kt_m = (c + r0 + 1) / kKeys;
  const int kt_a = max(0, min(kt_m - 1, nkt));
  for (int kt = kt0; kt < min(kt_a, kt1); ++kt) step(kt, std::false_type{});
  for (int kt = max(kt0, kt_a); kt < kt1; ++kt) step(kt, std::true_type{});

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (slot >= 0) {
    // a part: o relative to 2^m_run, its weight sum and m_run (rows with no key in this part
    // keep m_run = -1e30, l = 0, o = 0 and drop out of the merge)
    const size_t prow = ((size_t)slot * Hq + h) * kPrefillQTile + (my_row - r0);
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * mt + 8 * g4 + 4 * hl32;
        *reinterpret_cast<f32x4*>(po + d0) =
            f32x4{o[mt][4 * g4], o[mt][4 * g4 + 1], o[mt][4 * g4 + 2], o[mt][4 * g4 + 3]};
      }
    if (hl32 == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
    return;
  }
  const float inv = 1.f / l_tot;
  hl_bf16* op = attn_out + ((size_t)(qs + my_row) * Hq + h) * D;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * mt + 8 * g4 + 4 * hl32;
      const u32x2 v = {pack_bf2(o[mt][4 * g4] * inv, o[mt][4 * g4 + 1] * inv),
                       pack_bf2(o[mt][4 * g4 + 2] * inv, o[mt][4 * g4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + d0) = v;
    }
}

}  // namespace prefill
}  // namespace hl
