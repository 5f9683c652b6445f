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
// 32w..32w+31. Keys advance 32 at a time (two 16-token pages), staged through LDS (double
// buffered, register prefetch) and shared by the 4 waves. Scores are formed transposed,
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so each lane holds 16 keys of ONE query and the
// online-softmax max needs a single cross-lane exchange; P^T then feeds O^T = V^T P^T straight
// from registers (the k-slot order of the second product follows the register order of the
// first). V pages are stored dim-major ([d][16 tokens]) so the V^T operand is read without a
// transpose. Softmax runs in fp32 in the exp2 domain. Key tiles past a wave's last query are
// skipped; keys past a query's position are masked by select, and V rows past the sequence end
// are zeroed on load, so unused cache slots never reach the result.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 32;  // keys per tile = 2 pages

template <int D>
struct PrefillSmem {
  static constexpr int kRowBytes = D * 2;                 // one K row
  static constexpr int kKBytes = kKeys * kRowBytes;       // K tile [32][D]
  static constexpr int kVBytes = 2 * D * 32;              // V^T tile [2 pages][D][16]
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
};

// K tile: 16-byte chunk c of key row r lives at chunk c ^ (r & 7)
template <int D>
HL_DEV int k_off(int r, int c) {
  return r * (D * 2) + ((c ^ (r & 7)) << 4);
}
// V^T tile: 8-byte token quad q of dim row d (page pg) lives at quad q ^ ((d >> 2) & 3)
template <int D>
HL_DEV int v_off(int pg, int d, int q) {
  return pg * D * 32 + d * 32 + ((q ^ ((d >> 2) & 3)) << 3);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_attn_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ num_cached,
    const hl_bf16* __restrict__ q_rot, const hl_bf16* __restrict__ kpool,
    const hl_bf16* __restrict__ vpool, long long num_blocks, const int32_t* __restrict__ table,
    int max_blocks, const int32_t* __restrict__ tiles, int Hq, int Hkv, float scale_log2,
    hl_bf16* __restrict__ attn_out) {
  using SM = PrefillSmem<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int s = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int qs = q_start[s], n = q_start[s + 1] - qs, c = num_cached[s];
  const int kvh = h / (Hq / Hkv);
  const int kv_len = c + n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl32 = lane >> 5;
  const int tile_rows = min(128, n - r0);
  const int key_end = c + r0 + tile_rows;  // exclusive key bound of the whole tile
  const int nkt = (key_end + kKeys - 1) / kKeys;
  const int wr0 = r0 + 32 * wave;
  const int wave_key_end = c + min(wr0 + 32, n);  // exclusive; <= c + wr0 if the wave is empty
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

  // global -> register staging of one 32-key tile (K rows and V^T pages of head kvh)
  constexpr int kChunks = SM::kKBytes / 16;         // 16-byte chunks per K tile (= per V tile)
  constexpr int kPer = kChunks / kThreads;          // per thread: 2 for D = 128, 1 for D = 64
  constexpr int kChunksPerPage = kChunks / 2;
  u32x4 rk[kPer], rv[kPer];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + kThreads * i;
      const int pg = q / kChunksPerPage, w = q % kChunksPerPage;
      const int page = 2 * kt + pg;
      u32x4 kv4 = {0, 0, 0, 0}, vv4 = {0, 0, 0, 0};
      if (page * HL_BLOCK_SIZE < kv_len) {
        const int blk = trow[page];
        if (blk >= 0 && (long long)blk < num_blocks) {
          const size_t base = ((size_t)blk * Hkv + kvh) * page_elems;
          kv4 = *reinterpret_cast<const u32x4*>(kpool + base + (size_t)w * 8);
          vv4 = *reinterpret_cast<const u32x4*>(vpool + base + (size_t)w * 8);
          // V chunk w = dim row w / 2, tokens 8 (w & 1) .. +7; zero tokens past the end
          const int tok0 = page * HL_BLOCK_SIZE + 8 * (w & 1);
          if (tok0 + 8 > kv_len) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo_ok = (tok0 + 2 * e < kv_len) ? 0x0000ffffu : 0u;
              const uint32_t hi_ok = (tok0 + 2 * e + 1 < kv_len) ? 0xffff0000u : 0u;
              vv4[e] &= (lo_ok | hi_ok);
            }
          }
        }
      }
      rk[i] = kv4;
      rv[i] = vv4;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* kb = smem + buf * SM::kStage;
    uint8_t* vb = kb + SM::kKBytes;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + kThreads * i;
      const int pg = q / kChunksPerPage, w = q % kChunksPerPage;
      // K: page pg, row w / (D / 8), chunk w % (D / 8)
      const int r = pg * 16 + w / (D / 8), ch = w % (D / 8);
      *reinterpret_cast<u32x4*>(kb + k_off<D>(r, ch)) = rk[i];
      // V^T: page pg, dim row w / 2, token quads 2 (w & 1) and 2 (w & 1) + 1
      const int d = w >> 1, q0 = 2 * (w & 1);
      *reinterpret_cast<u32x2*>(vb + v_off<D>(pg, d, q0)) = u32x2{rv[i][0], rv[i][1]};
      *reinterpret_cast<u32x2*>(vb + v_off<D>(pg, d, q0 + 1)) = u32x2{rv[i][2], rv[i][3]};
    }
  };

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    sstore(buf);
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);
    if (kt * kKeys >= wave_key_end) continue;  // every key of this tile is after our queries
    const uint8_t* kb = smem + buf * SM::kStage;
    const uint8_t* vb = kb + SM::kKBytes;

    // S^T (32 keys x 32 queries)
    f32x16 st = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(kb + k_off<D>(lane & 31, 2 * ks + hl32));
      st = mfma32x32x16(ka, qf[ks], st);
    }
    // mask, scale, tile max; lane holds keys 8 (i / 4) + 4 hl32 + (i & 3) of its query
    float tmax = -1e30f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt * kKeys + 8 * (i >> 2) + 4 * hl32 + (i & 3);
      const float v = (key <= qpos) ? st[i] * scale_log2 : -INFINITY;
      st[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = wave_max_xor(tmax, 32);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2f(st[i] - m_new);
      st[i] = p;
      psum += p;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
    // P^T operand for page t: regs 8t .. 8t+7 (slot j <-> key 16t + 8 (j / 4) + 4 hl32 + j % 4)
    u32x4 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[t][e] = pack_bf2(st[8 * t + 2 * e], st[8 * t + 2 * e + 1]);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      const int d = 32 * mt + (lane & 31);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vb + v_off<D>(t, d, hl32));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vb + v_off<D>(t, d, 2 + hl32));
        o[mt] = mfma32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[t], o[mt]);
      }
    }
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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

}  // namespace

namespace hl {

hipError_t launch_prefill_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                    const int32_t* num_cached, const hl_bf16* q_rot,
                                    const hl_bf16* kpool, const hl_bf16* vpool,
                                    int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                                    const Plan& plan, hl_bf16* attn_out, hipStream_t st) {
  if (plan.n_pre_tiles <= 0) return hipSuccess;
  const float scale = cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(plan.n_pre_tiles, cfg.n_q_heads), block(kThreads);
  if (cfg.head_dim == 128) {
    hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, block, PrefillSmem<128>::kTotal, st,
                       q_start, num_cached, q_rot, kpool, vpool, (long long)num_blocks, table,
                       max_blocks, plan.pre_tiles, cfg.n_q_heads, cfg.n_kv_heads, scale_log2,
                       attn_out);
  } else {
    hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, block, PrefillSmem<64>::kTotal, st,
                       q_start, num_cached, q_rot, kpool, vpool, (long long)num_blocks, table,
                       max_blocks, plan.pre_tiles, cfg.n_q_heads, cfg.n_kv_heads, scale_log2,
                       attn_out);
  }
  return hipGetLastError();
}

}  // namespace hl
