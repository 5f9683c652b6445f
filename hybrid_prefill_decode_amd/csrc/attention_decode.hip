// Decode attention: one query row per sequence (qo_len = 1) over its long paged KV cache.
//
// Each decode reads only its own keys and values, so batching requests does not raise the
// arithmetic intensity: this phase is bound by HBM reads of the cache ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?"; "Gescheiden Prefill en Decode",
// section "Prefill versus Decode-prestaties"). The design therefore aims at streaming every K/V
// byte exactly once at full bandwidth:
//   * split-KV: a work unit is (sequence, run of `split_pages` pages, KV head); units are sized
//     from the batch so the grid holds thousands of workgroups whatever the length mix;
//   * all g = Hq / Hkv query heads of a KV head are served by each K/V read (GQA; head h reads
//     KV head h / g as in "7.8 Disaggregated Prefill/Decode & Chunked Prefill", GQA exercise);
//   * the 4 waves of a workgroup take alternate page pairs; every lane issues 16-byte K loads and
//     8-byte V loads that together cover each 4 KB page contiguously;
//   * the tiny products run on v_mfma_f32_16x16x32_bf16 with the page's 16 tokens as the M side:
//     S^T = K Q^T (columns = query heads) and O^T = V^T P^T, whose k-slot order is the register
//     order of S^T, so P never leaves registers; V pages are dim-major, so V^T is a plain load;
//   * q may come as two bf16 halves (q_rot + q_lo); the scores then take both products, which
//     costs nothing here (the matrix cores idle on this bandwidth-bound phase) and removes the
//     rounding of q from the result;
//   * softmax state (m, l, o) is fp32 in the exp2 domain; the waves' states are merged in LDS. A
//     sequence with one unit writes its row directly. Otherwise each unit writes a partial to the
//     workspace and a second kernel merges them (m* = max m_j, l* = sum l_j 2^(m_j - m*),
//     o = sum o_j 2^(m_j - m*) / l*), with the per-unit weights computed once in LDS and the
//     partial loads independent. (Merging in the last-finishing workgroup instead needs an
//     agent-scope release per workgroup, which writes back the XCD's L2 and costs more than the
//     extra launch.)
// Tokens past the sequence end are masked (scores by select, values zeroed on load).
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ num_cached,
    const hl_bf16* __restrict__ q_rot, const hl_bf16* __restrict__ q_lo,
    const hl_bf16* __restrict__ kpool, const hl_bf16* __restrict__ vpool, long long num_blocks,
    const int32_t* __restrict__ table, int max_blocks, const int32_t* __restrict__ units,
    const int32_t* __restrict__ dec_seqs, int split_pages,
    int Hq, int Hkv, float scale_log2, float* __restrict__ part, hl_bf16* __restrict__ attn_out) {
  __shared__ float sh_o[kWaves][D][16];
  __shared__ float sh_m[kWaves][16];
  __shared__ float sh_l[kWaves][16];
  // KV head fastest in dispatch order: the Hkv workgroups of a unit read the Hkv adjacent
  // 4 KB pieces of each block at about the same time
  const int kvh = blockIdx.x % Hkv, unit = blockIdx.x / Hkv;
  const int s = units[3 * unit], pg0 = units[3 * unit + 1], di = units[3 * unit + 2];
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
  auto load = [&](const int* blk, Pair& P) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool in = blk[h] >= 0 && (long long)blk[h] < num_blocks;
      const size_t base = ((size_t)(in ? blk[h] : 0) * Hkv + kvh) * page_elems;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        P.k[h][ks] = *reinterpret_cast<const u32x4*>(kpool + base + (size_t)col * D + 32 * ks + 8 * lg);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        P.v[h][mt] = *reinterpret_cast<const u32x2*>(vpool + base + (size_t)(16 * mt + col) * HL_BLOCK_SIZE + 4 * lg);
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

// Merge the split partials of each multi-unit decode sequence and write its attention row.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ dec_seqs,
    const float* __restrict__ part, int Hq, int Hkv, hl_bf16* __restrict__ attn_out) {
  __shared__ float sh_w[hl::kMaxUnitsPerSeq * 16];
  __shared__ float sh_mx[16], sh_lt[16];
  const int di = blockIdx.x, kvh = blockIdx.y;
  const int s = dec_seqs[3 * di], u0 = dec_seqs[3 * di + 1], nu = dec_seqs[3 * di + 2];
  if (nu == 1) return;  // written directly by the decode kernel
  const int g = Hq / Hkv;
  const int row = q_start[s];
  const int tid = threadIdx.x;
  const size_t ustride = (size_t)Hkv * g * (D + 2);
  const float* base = part + ((size_t)u0 * Hkv + kvh) * g * (D + 2);
  // m of every (unit, head) into LDS, then per-head max, weights and l*
  for (int e = tid; e < nu * g; e += kThreads) {
    const int u = e / g, hh = e - u * g;
    sh_w[u * 16 + hh] = base[u * ustride + hh * (D + 2) + D];
  }
  __syncthreads();
  if (tid < g) {
    float mx = -1e30f;
    for (int u = 0; u < nu; ++u) mx = fmaxf(mx, sh_w[u * 16 + tid]);
    sh_mx[tid] = mx;
  }
  __syncthreads();
  for (int e = tid; e < nu * g; e += kThreads) {
    const int u = e / g, hh = e - u * g;
    sh_w[u * 16 + hh] = exp2f(sh_w[u * 16 + hh] - sh_mx[hh]);
  }
  __syncthreads();
  if (tid < g) {
    float lt = 0.f;
    for (int u = 0; u < nu; ++u) lt += base[u * ustride + tid * (D + 2) + D + 1] * sh_w[u * 16 + tid];
    sh_lt[tid] = lt;
  }
  __syncthreads();
  for (int e = tid; e < g * D; e += kThreads) {
    const int hh = e / D, d = e - hh * D;
    const float* p = base + hh * (D + 2) + d;
    float acc = 0.f;
#pragma unroll 8
    for (int u = 0; u < nu; ++u) acc += p[u * ustride] * sh_w[u * 16 + hh];
    attn_out[((size_t)row * Hq + kvh * g + hh) * D + d] = (hl_bf16)f2bf(acc / sh_lt[hh]);
  }
}

}  // namespace

namespace hl {

hipError_t launch_decode_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                   const int32_t* num_cached, const hl_bf16* q_rot,
                                   const hl_bf16* q_lo,
                                   const hl_bf16* kpool, const hl_bf16* vpool,
                                   int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                                   const Plan& plan, hl_bf16* attn_out, hipStream_t st) {
  if (plan.n_dec_units <= 0) return hipSuccess;
  const float scale = cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(cfg.n_kv_heads * plan.n_dec_units), block(kThreads);
  if (cfg.head_dim == 128) {
    hipLaunchKernelGGL(decode_attn_kernel<128>, grid, block, 0, st, q_start, num_cached, q_rot,
                       q_lo, kpool, vpool, (long long)num_blocks, table, max_blocks, plan.dec_units,
                       plan.dec_seqs, plan.split_pages, cfg.n_q_heads,
                       cfg.n_kv_heads, scale_log2, plan.dec_part, attn_out);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(plan.n_dec_seqs, cfg.n_kv_heads), block, 0,
                       st, q_start, plan.dec_seqs, plan.dec_part, cfg.n_q_heads, cfg.n_kv_heads,
                       attn_out);
  } else {
    hipLaunchKernelGGL(decode_attn_kernel<64>, grid, block, 0, st, q_start, num_cached, q_rot,
                       q_lo, kpool, vpool, (long long)num_blocks, table, max_blocks, plan.dec_units,
                       plan.dec_seqs, plan.split_pages, cfg.n_q_heads,
                       cfg.n_kv_heads, scale_log2, plan.dec_part, attn_out);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(plan.n_dec_seqs, cfg.n_kv_heads), block, 0,
                       st, q_start, plan.dec_seqs, plan.dec_part, cfg.n_q_heads, cfg.n_kv_heads,
                       attn_out);
  }
  return hipGetLastError();
}

}  // namespace hl
