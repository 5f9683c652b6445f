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
#include "attn_decode_core.h"

namespace {

using hl::decode::kThreads;

// One workgroup per (unit, KV head), dispatched largest unit first when the plan orders the units
// so (Plan::dec_lpt, which shortens the launch's tail); KV head fastest, so the Hkv workgroups of
// a unit read the Hkv adjacent pieces of each block at about the same time. (Persistent workers
// that prefetch each next unit, as the fused launch can, were measured slower for this launch
// alone: the hardware's dispatch of one short-lived workgroup per unit already overlaps a unit's
// start with the streaming of the others on its compute unit.)
template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_kernel(hl::decode::DecodeArgs a,
                                                                  uint64_t* __restrict__ trace) {
  __shared__ hl::decode::DecodeLds<D> L;
  hl::decode::Carry<D> cy;
  cy.item = -1;
  cy.has_pair = false;
  const uint64_t t0 = trace ? (uint64_t)wall_clock64() : 0;
  // workgroups in rank order (largest unit first): rank r's unit sits at dec_position(r)
  const int units = a.n_items / a.Hkv, r = blockIdx.x / a.Hkv;
  const int item =
      a.lpt ? hl::dec_position(r, units) * a.Hkv + (blockIdx.x - r * a.Hkv) : (int)blockIdx.x;
  const int seq_item = hl::decode::decode_item<D, false>(a, item, L, cy);
  if (trace) {
    __syncthreads();
    hl::record_item(trace, seq_item, t0);
  }
}

// Merge the split partials of each multi-unit decode sequence and write its attention row.
// Two dependent rounds of loads: the (m, l) pairs of every unit and head (one 8-byte load each)
// together with the thread's o partials of the first kPre units, which do not depend on the
// weights; then one thread per head forms the max, the weights and l* from LDS. GMAX bounds the
// group size g (the thread's output elements live in registers); the LDS holds the batch's most
// units of one sequence (dynamic size: 2 * max units * g floats).
template <int D, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ dec_seqs,
    const float* __restrict__ part, int Hq, int Hkv, int max_units,
    hl_bf16* __restrict__ attn_out) {
  constexpr int kPre = 8;                                   // units whose o is loaded up front
  constexpr int kEl = (GMAX * D + kThreads - 1) / kThreads;  // output elements per thread
  extern __shared__ float sh[];
  __shared__ float sh_lt[16];
  const int di = blockIdx.x, kvh = blockIdx.y;
  const int s = dec_seqs[3 * di], u0 = dec_seqs[3 * di + 1], nu = dec_seqs[3 * di + 2];
  if (nu == 1) return;  // written directly by the decode kernel
  const int g = Hq / Hkv;
  float* sh_w = sh;                   // [max_units][g]: m, then the weights 2^(m - m*)
  float* sh_l = sh + max_units * g;   // [max_units][g]
  const int tid = threadIdx.x;
  const size_t ustride = (size_t)Hkv * g * (D + 2);
  const float* base = part + ((size_t)u0 * Hkv + kvh) * g * (D + 2);
  float pre[kEl][kPre];
#pragma unroll
  for (int i = 0; i < kEl; ++i) {
    const int e = tid + i * kThreads;
    const int hh = e / D, d = e - hh * D;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      pre[i][u] = (e < g * D && u < nu) ? base[u * ustride + hh * (D + 2) + d] : 0.f;
  }
  for (int e = tid; e < nu * g; e += kThreads) {
    const int u = e / g, hh = e - u * g;
    const float2 ml = *reinterpret_cast<const float2*>(base + u * ustride + hh * (D + 2) + D);
    sh_w[u * g + hh] = ml.x;
    sh_l[u * g + hh] = ml.y;
  }
  const int row = q_start[s];
  __syncthreads();
  if (tid < g) {
    float mx = -1e30f;
    for (int u = 0; u < nu; ++u) mx = fmaxf(mx, sh_w[u * g + tid]);
    float lt = 0.f;
    for (int u = 0; u < nu; ++u) {
      const float w = exp2f(sh_w[u * g + tid] - mx);
      sh_w[u * g + tid] = w;
      lt += sh_l[u * g + tid] * w;
    }
    sh_lt[tid] = lt;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kEl; ++i) {
    const int e = tid + i * kThreads;
    if (e >= g * D) break;
    const int hh = e / D, d = e - hh * D;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (u < nu) acc += pre[i][u] * sh_w[u * g + hh];
    const float* p = base + hh * (D + 2) + d;
    for (int u = kPre; u < nu; ++u) acc += p[u * ustride] * sh_w[u * g + hh];
    attn_out[((size_t)row * Hq + kvh * g + hh) * D + d] = (hl_bf16)f2bf(acc / sh_lt[hh]);
  }
}

}  // namespace

namespace hl {

using decode::kThreads;

hipError_t launch_decode_merge(const hl_layer_cfg& cfg, const int32_t* q_start, const Plan& plan,
                               hl_bf16* attn_out, hipStream_t st) {
  if (plan.n_dec_seqs <= 0) return hipSuccess;
  const dim3 grid(plan.n_dec_seqs, cfg.n_kv_heads), block(kThreads);
  const int g = cfg.n_q_heads / cfg.n_kv_heads;
  const int mu = plan.max_seq_units > 0 ? plan.max_seq_units : hl::kMaxUnitsPerSeq;
  const size_t lds = sizeof(float) * 2 * (size_t)mu * g;
  auto kernel = cfg.head_dim == 128
                    ? (g <= 8 ? decode_merge_kernel<128, 8> : decode_merge_kernel<128, 16>)
                    : (g <= 8 ? decode_merge_kernel<64, 8> : decode_merge_kernel<64, 16>);
  hipLaunchKernelGGL(kernel, grid, block, lds, st, q_start, plan.dec_seqs, plan.dec_part,
                     cfg.n_q_heads, cfg.n_kv_heads, mu, attn_out);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                   const int32_t* num_cached, const hl_bf16* q_rot,
                                   const hl_bf16* q_lo, const hl_bf16* kpool,
                                   const hl_bf16* vpool, int64_t num_blocks, const int32_t* table,
                                   int32_t max_blocks, const Plan& plan, int32_t cus,
                                   hl_bf16* attn_out, hipStream_t st) {
  (void)cus;
  if (plan.n_dec_units <= 0) return hipSuccess;
  const float scale =
      cfg.softmax_scale > 0.f ? cfg.softmax_scale : 1.f / sqrtf((float)cfg.head_dim);
  const dim3 grid(cfg.n_kv_heads * plan.n_dec_units), block(kThreads);
  const decode::DecodeArgs args{q_start,          num_cached,  q_rot,      q_lo,
                                kpool,            vpool,       (long long)num_blocks, table,
                                max_blocks,       plan.dec_units, plan.dec_seqs, plan.split_pages,
                                cfg.n_q_heads,    cfg.n_kv_heads, scale * 1.4426950408889634f,
                                plan.dec_part,    attn_out,    plan.n_dec_units * cfg.n_kv_heads,
                                plan.dec_lpt};
  // decode records follow the batch's prefill records in the trace
  uint64_t* trace =
      plan.trace ? plan.trace + 3 * (size_t)plan.n_pre_tiles * cfg.n_q_heads : nullptr;
  if (cfg.head_dim == 128)
    hipLaunchKernelGGL(decode_attn_kernel<128>, grid, block, 0, st, args, trace);
  else
    hipLaunchKernelGGL(decode_attn_kernel<64>, grid, block, 0, st, args, trace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(cfg, q_start, plan, attn_out, st);
}

}  // namespace hl
