// Device-side primitives shared by the gfx950 kernels of the hybrid layer step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "hybrid_layer.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define HL_DEV __device__ __forceinline__

// Element offset, inside one (block, KV head) K page, of elements 8c .. 8c+7 of the page's token
// t. K pages are chunk-major, [head_dim / 8][16 tokens][8]: the same 16-byte chunk of the 16
// tokens is one contiguous 256-byte run, so a wave's K fragment load for a matrix-core step
// (16 tokens x 4 chunks) reads 1 KB contiguously instead of sixteen 64-byte pieces 256 bytes apart.
__host__ __device__ constexpr int kpage_off(int t, int c) { return (c * 16 + t) * 8; }

// bf16 <-> fp32. bf16 is the top half of an fp32. Narrowing uses the CDNA4 packed conversion
// (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN), one instruction for two values.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
HL_DEV float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
HL_DEV float bf_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
HL_DEV float bf_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
HL_DEV uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
HL_DEV uint32_t f2bf(float f) { return pack_bf2(f, 0.f) & 0xffffu; }

HL_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Matrix-core products (CDNA4): D = A B + C with 8 bf16 of A and of B per lane.
HL_DEV f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
HL_DEV f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32). Softmax weights use it with x <= 8; results
// below 2^-126 may flush to zero, a change below 2^-126 relative to the largest weight.
HL_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// c + a.lo * b.lo + a.hi * b.hi over bf16 pairs, accumulated in fp32 (v_dot2_f32_bf16)
HL_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// Non-temporal store (written through without staying dirty in the caches). For the QKV
// projection's outputs (rotated q, its low half, the appended K/V rows), which attention reads
// next: lines left dirty in the memory-side cache are written back while attention streams the
// KV pools, and measured about 1 us of that launch per MB (70B-shaped batch: -30 us). Data the
// very next GEMM reads (the normed activations) keeps plain stores: written through, the GEMM
// fetched it from HBM and ran ~5 us slower.
template <class T>
HL_DEV void store_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }
HL_DEV float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
HL_DEV float wave_sum_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

// Internal launchers (each returns hipSuccess or the launch error).
namespace hl {

constexpr int kPrefillQTile = 128;   // query rows per prefill work tile
constexpr int kPrefillKeyTile = 64;  // keys per step of a prefill work item
constexpr int kPreEntry = 5;         // ints per prefill work entry (see Plan::pre_tiles)

// Key tiles a prefill tile of `rows` query rows from row r0 of a chunk after c cached tokens
// reads (causal: up to its last row's position), and the parts it is split into when a part
// holds at most `split` key tiles. Host and plan kernel count work with these same functions.
__host__ __device__ inline int prefill_key_tiles(int c, int r0, int rows) {
  return (c + r0 + rows + kPrefillKeyTile - 1) / kPrefillKeyTile;
}
__host__ __device__ inline int prefill_parts(int key_tiles, int split) {
  return (key_tiles + split - 1) / split;
}

// Prefill work item (entry * Hq + query head) at position p of the dispatch order. The launches
// hand each of the 8 XCDs a contiguous run of positions; the order deals the items to 8 sections
// in units of one entry and one KV head (its Hq / Hkv query heads, which read the same K/V
// tiles): unit u = entry * Hkv + kv head goes to section u % 8, each section keeping the entries'
// order (longest key range first). With 8 KV heads every section is one KV head over all entries,
// so the XCDs get equal work and each streams one head's keys and values through its own L2.
__host__ __device__ inline int prefill_item_at(int p, int n_ent, int Hq, int Hkv) {
  const int g = Hq / Hkv, n_units = n_ent * Hkv;
  for (int x = 0; x < 8; ++x) {
    const int here = (x < n_units ? (n_units - x + 7) / 8 : 0) * g;
    if (p < here) {
      const int u = x + 8 * (p / g);
      return (u / Hkv) * Hq + (u % Hkv) * g + p % g;
    }
    p -= here;
  }
  return -1;  // p out of range
}

constexpr int kDecUnitInts = 16;

// Dispatch order of the decode units (when Plan::dec_lpt): largest first, so the last units of a
// launch are short and the workers run out of work at nearly the same time
// (longest-processing-time-first list scheduling). Full units (split_pages pages) take ranks 0..F-1 in sequence order; each sequence's
// last unit, when shorter, goes into one of kDecBuckets size classes, the longer classes first.
constexpr int kDecBuckets = 8;
// size class of a last unit of `rem` pages, 0 < rem < split (larger class = longer unit)
__host__ __device__ inline int dec_bucket(int rem, int split) {
  return (rem * kDecBuckets - 1) / split;
}
// Position in the unit list of the unit of rank r among n: the ranks are dealt round-robin to 8
// contiguous runs of positions (the fused launch's per-XCD queues), so each run holds every 8th
// rank, largest first.
__host__ __device__ inline int dec_position(int r, int n) {
  const int x = r & 7, rem = n & 7;
  return x * (n >> 3) + (x < rem ? x : rem) + (r >> 3);
}

struct Plan {
  // device work lists inside the workspace
  int32_t* dec_units;      // [n_dec_units][kDecUnitInts] in dispatch order (dec_position):
                           // (seq, first page, decode index, units of the sequence, its query
                           // row, its KV length, partial slot, 0, then the block ids of its pages
                           // first .. first + 7, clamped to its last page): everything a unit's
                           // first page pairs need, in one 64-byte record. The partial slot is
                           // the unit's index in sequence order (dec_seqs and dec_part use it);
                           // without dec_lpt the records are in that order too.
  int32_t* dec_seqs;       // [n_dec_seqs][3]: (seq, first unit, unit count)
  int32_t* pre_tiles;      // [n_pre_tiles][kPreEntry]: (seq, first query row within the sequence,
                           // first key tile, end key tile, partial slot or -1 if unsplit)
  int32_t* pre_merge;      // [n_pre_merge][4]: (seq, first query row, first slot, part count)
  float* dec_part;         // [n_dec_units][Hkv][group][head_dim + 2] partial (o, m, l)
  float* pre_part_o;       // [slots][Hq][kPrefillQTile][head_dim] unnormalised partial o
  float2* pre_part_ml;     // [slots][Hq][kPrefillQTile] partial (m, l)
  int32_t* counters;       // [kPlanCounters][kCounterStride] work-queue counters of the fused
                           // attention kernel (one per 256-byte line), zeroed by the plan kernel
  int32_t n_dec_units, n_dec_seqs, n_pre_tiles, n_pre_merge;
  int32_t split_pages;     // pages per decode work unit
  int32_t dec_rank_base[kDecBuckets];  // first rank of each size class of last units
  int32_t dec_lpt = 0;     // 1: dec_units in largest-first dispatch order, 0: in sequence order
  int32_t max_seq_units = 0;  // most decode units of one sequence (sizes the merge's LDS)
  int32_t pre_split;       // key tiles per prefill work part
  bool fused_prefetch = false;  // fused launch: decode units prefetch the next (decode-heavy)
  uint64_t* trace = nullptr;  // optional [items][3]: (start, end, worker) of every work item,
                              // prefill items first, then decode units (see record_item)
};

// Trace record of one work item: its start and end on the device's constant-rate clock and the
// workgroup that ran it. Thread 0 writes it once the whole workgroup has finished the item.
HL_DEV void record_item(uint64_t* trace, int item, uint64_t t0) {
  if (threadIdx.x == 0) {
    uint64_t* r = trace + 3 * (size_t)item;
    r[0] = t0;
    r[1] = (uint64_t)wall_clock64();
    r[2] = blockIdx.x;
  }
}

// Per-token data of one step (filled by the first prep pass, read by the QKV GEMM epilogue).
constexpr int32_t kDecodeBit = 1 << 30;  // positions are below 2^30 (checked on the host)
struct TokenInfo {
  const int32_t* q_start;
  const int32_t* num_cached;
  int32_t num_seqs;
  const int32_t* table;
  int32_t max_blocks;
  int64_t num_blocks;
  int32_t head_dim;
  float rope_theta;
  int32_t* tok_pos;   // [T] absolute position, | kDecodeBit for a decode token (q_len == 1)
  int32_t* tok_blk;   // [T] physical block of that position (-1 if out of range)
  float2* rope_cs;    // [T][head_dim / 2] (cos, sin)
};

// Epilogue of the token-batched GEMM.
constexpr int kEpiRopeAppend = 3;  // internal: rotate q/k, write q_rot and the K/V pages
struct GemmEpi {
  int32_t kind;               // HL_EPI_NONE / RESIDUAL / SWIGLU / kEpiRopeAppend
  const hl_bf16* residual;    // RESIDUAL: [m, n]
  const float* row_scale;     // optional [m]: acc *= row_scale[row] before the epilogue math
  // kEpiRopeAppend
  int32_t n_q_heads, n_kv_heads, head_dim;
  hl_bf16* q_rot;
  hl_bf16* q_lo;              // optional: bf16(q - bf16(q)), the rounding residue of q_rot
  hl_bf16* kpool;
  hl_bf16* vpool;
  const int32_t* tok_pos;
  const int32_t* tok_blk;
  const float2* rope_cs;
};

// plan: also build the attention work lists (kPlanWorkgroups extra workgroups; needs ti).
hipError_t launch_prep(const hl_bf16* x, const hl_bf16* gain, hl_bf16* xg, float* rscale,
                       int32_t rows, int32_t cols, float eps, const TokenInfo* ti,
                       hipStream_t st, const Plan* plan = nullptr);
hipError_t launch_plan(const int32_t* q_start, const int32_t* num_cached, int32_t num_seqs,
                       const int32_t* table, int32_t max_blocks, const Plan& plan,
                       hipStream_t st);
constexpr int kPlanCounters = 16;
constexpr int kPlanWorkgroups = 8;  // workgroups that build the work lists together
constexpr int kCounterStride = 64;  // int32 slots per counter: each on its own 256-byte line
constexpr int kMaxUnitsPerSeq = 256;  // decode work units of one sequence (merge weights in LDS)
hipError_t launch_rmsnorm(const hl_bf16* x, const hl_bf16* g, hl_bf16* y, int32_t rows,
                          int32_t cols, float eps, hipStream_t st);
hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t st);
size_t gemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t epi);
struct TileChoice {
  int bm, bn;
  bool sk;            // stream-K (plain and residual epilogues with a workspace only)
  int splits = 0;     // >= 2: split-K into that many K ranges (SwiGLU and RoPE epilogues)
  bool tail = false;  // with splits: one tile per workgroup, but the tiles past the last full
                      // round over the compute units are split into `splits` K ranges
};
// Schedules a launch may use besides one tile per workgroup (each needs the workspace).
constexpr int kSchedStreamK = 1, kSchedSplitK = 2, kSchedTail = 4;
// split-K on the 256-wide tiles too, priced at the k-step cost of a one-tile run (plain and
// residual epilogues: measured faster there, slower for SwiGLU and RoPE)
constexpr int kSchedWideSplit = 8;
// the 192-wide tiles (SwiGLU epilogue only, one tile per workgroup)
constexpr int kSchedSwigluTiles = 16;
// Tile shape and schedule of a GEMM launch (gemm.hip); col_align: N-tile widths a multiple of it.
TileChoice choose_tiles(int m, int n, int k, int schedules, int col_align);
bool gemm_tile_supported(int bm, int bn, int epilogue, int stream_k);
bool gemm_split_fits(int m, int n, int bm, int bn, int splits);  // pieces fit the workspace
bool gemm_tail_fits(int m, int n, int bm, int bn, int splits);  // tail-split pieces fit it
// few-token path (gemm_skinny.hip): split-K weight streaming with fp32 partials in the workspace
constexpr int kSkinnyMaxM = 64;
size_t skinny_workspace_bytes(int m, int n, int k);
bool use_skinny(int m, int n, int k, size_t ws_bytes);  // the path launch_gemm takes
hipError_t launch_gemm_skinny(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                              const GemmEpi& epi, float* part, hipStream_t st);
// plain / residual / SwiGLU GEMM with a given tile shape (stream-K needs the workspace)
hipError_t launch_gemm_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                             int32_t k, const GemmEpi& epi, const TileChoice& tc, void* ws,
                             hipStream_t st);
hipError_t launch_rope_append(const hl_layer_cfg& cfg, int32_t num_seqs, int32_t num_tokens,
                              const int32_t* q_start, const int32_t* num_cached,
                              const hl_bf16* qkv, hl_bf16* q_rot, hl_bf16* kpool,
                              hl_bf16* vpool, int64_t num_blocks, const int32_t* table,
                              int32_t max_blocks, hipStream_t st);
hipError_t launch_prefill_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                    const int32_t* num_cached, const hl_bf16* q_rot,
                                    const hl_bf16* kpool, const hl_bf16* vpool,
                                    int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                                    const Plan& plan, hl_bf16* attn_out, hipStream_t st);
hipError_t launch_decode_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                   const int32_t* num_cached, const hl_bf16* q_rot,
                                   const hl_bf16* q_lo,
                                   const hl_bf16* kpool, const hl_bf16* vpool,
                                   int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                                   const Plan& plan, int32_t cus, hl_bf16* attn_out,
                                   hipStream_t st);

hipError_t launch_decode_merge(const hl_layer_cfg& cfg, const int32_t* q_start, const Plan& plan,
                               hl_bf16* attn_out, hipStream_t st);
hipError_t launch_prefill_merge(const hl_layer_cfg& cfg, const int32_t* q_start, const Plan& plan,
                                hl_bf16* attn_out, hipStream_t st);
// Prefill and decode attention of one batch in a single launch (plus the decode merge); `cus`
// is the device's compute-unit count.
hipError_t launch_hybrid_attention(const hl_layer_cfg& cfg, const int32_t* q_start,
                                   const int32_t* num_cached, const hl_bf16* q_rot,
                                   const hl_bf16* q_lo, const hl_bf16* kpool,
                                   const hl_bf16* vpool, int64_t num_blocks, const int32_t* table,
                                   int32_t max_blocks, const Plan& plan, int32_t cus,
                                   hl_bf16* attn_out, hipStream_t st);

// Model-level kernels (model.hip).
hipError_t launch_embed(const int32_t* tokens, const hl_bf16* table, hl_bf16* x, int T, int H,
                        int vocab, hipStream_t st);
hipError_t launch_last_rows(const int32_t* q_start, const hl_bf16* x, hl_bf16* rows, int S, int H,
                            hipStream_t st);
hipError_t launch_argmax(const hl_bf16* logits, int S, int V, int32_t* out, hipStream_t st);

// One request's K/V span to (exporting) or from the [L][2][T][Hkv][d] transfer layout.
hipError_t launch_kv_span(const hl_kv_span& s, const hl_kv_pages& kv, hl_bf16* buf, bool exporting);

}  // namespace hl
