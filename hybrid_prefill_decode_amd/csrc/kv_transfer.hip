// One request's paged K/V to and from the transfer layout [L][2][T][Hkv][d].
//
// A prefill instance hands a finished prompt's KV cache to a decode instance as one tensor of
// shape [layers, 2 (K, V), tokens, KV heads, head dim], which the decode instance places into its
// own paged cache ("7.8 Disaggregated Prefill/Decode & Chunked Prefill", "Lifecycle of a
// Request"); the copy runs layer by layer, each layer's slice as soon as that layer has appended
// its rows, so all but the last layer's transfer hides under the prefill compute ("Layer-Wise
// Pipelining"). These kernels are the GPU side of one such layer slice on one device: export
// gathers the request's pages into the contiguous slice (what a peer copy or an RDMA write then
// moves in one piece), import scatters a received slice into pages of another block table.
//
// One workgroup per (page of the span, KV head), 2 d threads. Each thread moves one 16-byte chunk
// of one token's K row between the slice and the page (chunk-major: chunk c of token t sits at
// (c * 16 + t) * 8 elements into the page). V pages are dim-major (each
// (block, head) page is one contiguous run, as "Gescheiden Prefill en Decode" asks for sharded
// transfers), so V goes through an LDS transpose: the page is read (or written) in 16-byte
// pieces of a dim row, the slice in 16-byte pieces of a token row. Slots outside the span are
// never written: export skips them; import writes K chunks of in-span tokens only and rewrites a
// partial V page only after reading it, so its other tokens keep their bytes.
#include "common.h"

namespace {

template <int D>
struct SpanArgs {
  const int32_t* table;
  int start, count, Hkv;
  uint32_t num_blocks;
  hl_bf16* kpool;
  hl_bf16* vpool;
  hl_bf16* kslab;  // [count][Hkv][D] of this layer
  hl_bf16* vslab;
};

// LDS transpose of one V page: [16 tokens][D + 8] bf16 (the pad keeps rows 16-byte aligned and
// spreads the column accesses over banks)
template <int D>
struct VStage {
  uint16_t t[16][D + 8];
};

template <int D, bool EXPORT>
__global__ __launch_bounds__(2 * D) void kv_span_kernel(SpanArgs<D> a) {
  __shared__ __attribute__((aligned(16))) VStage<D> vs;
  constexpr int CH = D / 8;  // 16-byte chunks per token row
  const int lp = a.start / HL_BLOCK_SIZE + (int)blockIdx.x;  // logical page
  const int h = blockIdx.y;
  const uint32_t raw = (uint32_t)a.table[lp];
  const uint32_t b = raw < a.num_blocks ? raw : 0u;  // validated on the host; never out of bounds
  const int tid = threadIdx.x;
  const size_t page = ((size_t)b * a.Hkv + h) * HL_BLOCK_SIZE * D;
  // token-row view: token tok of the page, chunk ch
  const int tok = tid / CH, ch = tid % CH;
  const int p = lp * HL_BLOCK_SIZE + tok;
  const bool in = p >= a.start && p < a.start + a.count;
  const size_t srow = ((size_t)(p - a.start) * a.Hkv + h) * D + 8 * ch;
  // dim-row view of the V page: dim r, tokens 8 half .. 8 half + 7
  const int r = tid >> 1, half = tid & 1;
  u32x4* kp = reinterpret_cast<u32x4*>(a.kpool + page + kpage_off(tok, ch));
  u32x4* vp = reinterpret_cast<u32x4*>(a.vpool + page + (size_t)r * HL_BLOCK_SIZE + 8 * half);
  const int p0 = lp * HL_BLOCK_SIZE;
  const bool whole = p0 >= a.start && p0 + HL_BLOCK_SIZE <= a.start + a.count;
  if constexpr (EXPORT) {
    const u32x4 kv = *kp, v = *vp;
    if (in) *reinterpret_cast<u32x4*>(a.kslab + srow) = kv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vs.t[8 * half + 2 * j][r] = (uint16_t)(v[j] & 0xffffu);
      vs.t[8 * half + 2 * j + 1][r] = (uint16_t)(v[j] >> 16);
    }
    __syncthreads();
    if (in) *reinterpret_cast<u32x4*>(a.vslab + srow) = *reinterpret_cast<const u32x4*>(&vs.t[tok][8 * ch]);
  } else {
    // both slice loads first (and the page, if only part of it is replaced), then the stores
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (in) {
      kv = *reinterpret_cast<const u32x4*>(a.kslab + srow);
      vv = *reinterpret_cast<const u32x4*>(a.vslab + srow);
    }
    u32x4 old = {0u, 0u, 0u, 0u};
    if (!whole) old = *vp;  // a partial page keeps its other tokens
    if (in) *kp = kv;
    *reinterpret_cast<u32x4*>(&vs.t[tok][8 * ch]) = vv;
    __syncthreads();
    // tokens 8 half .. 8 half + 7 of dim r; out-of-span tokens keep the old bits (their LDS
    // entries were not written and are not used)
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q0 = p0 + 8 * half + 2 * e;
      const uint32_t lo = vs.t[8 * half + 2 * e][r], hi = vs.t[8 * half + 2 * e + 1][r];
      const bool in0 = q0 >= a.start && q0 < a.start + a.count;
      const bool in1 = q0 + 1 >= a.start && q0 + 1 < a.start + a.count;
      v[e] = (in0 ? lo : (old[e] & 0xffffu)) | ((in1 ? hi : (old[e] >> 16)) << 16);
    }
    *vp = v;
  }
}

template <int D, bool EXPORT>
hipError_t launch_span(const hl_kv_span& s, const hl_kv_pages& kv, hl_bf16* buf) {
  const int first = s.start / HL_BLOCK_SIZE, last = (s.start + s.count - 1) / HL_BLOCK_SIZE;
  SpanArgs<D> a;
  a.table = s.table;
  a.start = s.start;
  a.count = s.count;
  a.Hkv = s.n_kv_heads;
  a.num_blocks = (uint32_t)std::min<int64_t>(kv.num_blocks, (int64_t)UINT32_MAX);
  a.kpool = kv.k;
  a.vpool = kv.v;
  const size_t slab = (size_t)s.count * s.n_kv_heads * D;
  a.kslab = buf + (size_t)s.layer * 2 * slab;
  a.vslab = a.kslab + slab;
  hipLaunchKernelGGL((kv_span_kernel<D, EXPORT>), dim3(last - first + 1, s.n_kv_heads),
                     dim3(2 * D), 0, static_cast<hipStream_t>(s.stream), a);
  return hipGetLastError();
}

}  // namespace

namespace hl {

hipError_t launch_kv_span(const hl_kv_span& s, const hl_kv_pages& kv, hl_bf16* buf, bool exporting) {
  if (s.count == 0) return hipSuccess;
  if (s.head_dim == 128)
    return exporting ? launch_span<128, true>(s, kv, buf) : launch_span<128, false>(s, kv, buf);
  return exporting ? launch_span<64, true>(s, kv, buf) : launch_span<64, false>(s, kv, buf);
}

}  // namespace hl
