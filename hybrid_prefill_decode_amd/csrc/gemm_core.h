// Token-batched linear layer on the CDNA4 matrix cores: C = A W^T (bf16 in, fp32 accumulate).
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?").
//
// Main loop (256 threads = 4 waves, one per SIMD; K advances 64 per tile, in two k32 steps). Each
// wave owns a (BM/2) x (BN/2) block of 16 x 16 v_mfma_f32_16x16x32_bf16 outputs whose fp32
// accumulators live in the accumulation registers (256 of them for a 256 x 256 tile), so the 256
// ordinary registers stay free for fragments and staging. (On gfx950 the 16 x 16 x 32 form sustains
// about 13 % more bf16 throughput on random operands than 32 x 32 x 16, measured with the same wave
// tile and LDS traffic.) A and W tiles are staged through LDS in 128-byte rows whose 16-byte chunks
// are XOR-swizzled with (row / 2) mod 8, which keeps every 16-lane group of a fragment read on
// distinct banks. Per tile: k32 step 0 carries the fragment reads of step 1 and all of the tile's
// staging work (LDS writes of tile t+1 from registers, global loads of tile t+2 into them), spread
// evenly over its MFMAs in an order pinned with sched_barrier; the barrier sits before step 1,
// whose MFMAs hide the fragment reads of the next tile's step 0. Fragment reads go in the order
// the next step first uses them (W blocks, then A blocks, each A block only after the current
// step's last use of it), so the A fragments need a single register set.
// Tiles are dealt so that consecutive tile ids land on the same XCD (workgroups go to the 8 XCDs
// round-robin) and, within an XCD, the M tiles of one N column run together, so a weight tile is
// fetched from HBM once.
//
// Schedules. Wide GEMMs run one tile per workgroup. Narrow ones (N = hidden for the O and down
// projections leaves fewer tiles than compute units) run stream-K: exactly one workgroup per CU,
// each taking an equal run of (tile, k-step) iterations; a tile split between workgroups is written
// as fp32 pieces to the workspace and finished by a fix-up kernel that sums the pieces and applies
// the epilogue. The SwiGLU and RoPE epilogues need a whole tile (gate and up columns together,
// whole heads), so when their tiles are too few to fill the compute units (a batch of a few
// hundred tokens) they run split-K instead: workgroup (tile, s) takes the s-th of S equal K
// ranges and writes its fp32 accumulators as a piece; the fix-up sums the S pieces in order and
// applies the epilogue.
//
// Epilogues, after an optional per-row scale (the RMSNorm factor, see prep.hip): plain, + residual,
// SwiGLU (the W tile holds BN/2 gate rows and the matching BN/2 up rows; a lane holds a gate and
// its up in registers), and RoPE + KV append for the QKV projection (the fp32 tile is staged in
// LDS; q heads are rotated into q_rot, k heads rotated and v heads copied into their cache pages).
#pragma once
#include "common.h"

namespace hl {
// One translation unit per epilogue (compiled in parallel): gemm_<epilogue>.hip.
hipError_t launch_gemm_plain(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                             int m, int n, int k, const GemmEpi& epi, float* part, hipStream_t st);
hipError_t launch_gemm_residual(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w,
                                hl_bf16* c, int m, int n, int k, const GemmEpi& epi, float* part,
                                hipStream_t st);
hipError_t launch_gemm_swiglu(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                              int m, int n, int k, const GemmEpi& epi, float* part,
                              hipStream_t st);
hipError_t launch_gemm_rope(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                            int m, int n, int k, const GemmEpi& epi, float* part, hipStream_t st);
}  // namespace hl

namespace {
using hl::GemmEpi;
using hl::kEpiRopeAppend;

constexpr int BK = 64, kThreads = 256;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format; no swizzle, no stride)
constexpr int kBufferFlags = 0x00020000;
// stream-K: one workgroup per compute unit, each with up to two fp32 pieces of a 256 x 256 tile
constexpr int kStreamKGrid = 256;
constexpr size_t kStreamKWorkspace = (size_t)kStreamKGrid * 2 * 256 * 256 * 4;

// 128-byte LDS rows (64 bf16 of K); 16-byte chunk c of row r lives at chunk c ^ ((r >> 1) & 7)
HL_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Bijection from dispatch order to tile order that keeps consecutive tiles on one XCD.
HL_DEV int xcd_tile(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

HL_DEV float silu(float g) { return g / (1.f + __expf(-g)); }

struct Sched {
  int mtiles, ntiles, nk;  // tiles in M and N; k-steps per tile
  int ipw;                 // stream-K: k-steps per workgroup (0: one tile per workgroup)
  int phase_runs;          // stream-K: run = dispatch index (else XCD-contiguous runs)
  float* part;             // stream-K: [grid][2][BM * BN] fp32 pieces
};

template <int BM, int BN>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
  static constexpr int MT = WM / 16, NT = WN / 16;  // 16 x 16 output blocks of one wave
  static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int A_CH = A_BYTES / 16 / kThreads, W_CH = W_BYTES / 16 / kThreads;
  static constexpr int NCH = A_CH + W_CH;
  static constexpr int MAIN_LDS = 2 * STAGE;
  static_assert(A_CH * kThreads * 16 == A_BYTES && W_CH * kThreads * 16 == W_BYTES, "staging");
};

// Load depth of the one-tile main loop (k-steps from a tile's load to its use). The 128-wide
// tiles have the shortest k-steps and take their weights from HBM in a model iteration, so their
// loads get an extra k-step in flight.
template <int BM, int BN>
constexpr int kLoadDepth = (BN == 128 || (BN == 192 && BM <= 128)) ? 3 : 2;

// fp32 row stride (floats) of the RoPE epilogue's LDS stage of a BN-wide tile
template <int BN>
constexpr int kStageRow = BN + 4;

// Row of the W tile that feeds block t of wave column wn (SwiGLU pairs gate block t with up
// block t + NT/2 so both land in the same lane).
template <int EPI, int BN, int WN, int NT>
HL_DEV int w_block_row(int wn, int t) {
  if (EPI == HL_EPI_SWIGLU)
    return (t < NT / 2) ? wn * (WN / 2) + t * 16 : BN / 2 + wn * (WN / 2) + (t - NT / 2) * 16;
  return wn * WN + t * 16;
}

// Issue slots of a step's NM MFMAs: staging pair i follows MFMA i NM / NCH, fragment read j
// follows MFMA (j + 1) NM / NR - 1 (both maps are one-to-one since NM >= NCH, NR). -1: none.
constexpr int stage_after(int q, int nm, int nch) {
  const int i = (q * nch + nm - 1) / nm;
  return (i < nch && (i * nm) / nch == q) ? i : -1;
}
constexpr int read_after(int q, int nm, int nr) {
  const int j = ((q + 1) * nr + nm - 1) / nm - 1;
  return (j >= 0 && j < nr && ((j + 1) * nm) / nr - 1 == q) ? j : -1;
}

// One tile's K range [kb, ke) into acc (acc zeroed here).
template <int EPI, int BM, int BN, int D = kLoadDepth<BM, BN>, bool MC = BN != 256>
HL_DEV void mainloop(const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, int M, int N,
                     int K, int mt, int nt, int kb, int ke, uint8_t* smem,
                     f32x4 (&acc)[Cfg<BM, BN>::MT][Cfg<BM, BN>::NT]) {
  using C = Cfg<BM, BN>;
  constexpr int MT = C::MT, NT = C::NT, NCH = C::NCH, A_CH = C::A_CH;
  constexpr int NM = MT * NT, NR = MT + NT, KS = BK / 32;  // MFMAs and fragment reads per step
  static_assert(KS == 2, "the W fragment sets alternate per step and must line up across tiles");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = mt * BM;
  const int half_n = N >> 1;

  // Staging: chunk i of a thread is row (tid / 8) + 32 i of the A tile (i < A_CH) or of the W
  // tile, 16-byte column tid % 8. Rows past M read row M-1: a C row depends only on its own A
  // row and padded C rows are never stored, so the loads need no branch. Loads are buffer loads:
  // a 32-bit per-thread byte offset (the host bounds M K and N K below 2^31 elements) plus a
  // workgroup-uniform one (k, and the W rows of the tile) in a scalar register, so the 16 loads
  // of a tile cost 9 address registers instead of 16 64-bit pointers.
  const int srow = tid >> 3, sch8 = (tid & 7) * 8;
  const __amdgpu_buffer_rsrc_t rs_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<hl_bf16*>(A), 0, (int)((uint32_t)M * (uint32_t)K * 2u), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_w =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<hl_bf16*>(W), 0, (int)((uint32_t)N * (uint32_t)K * 2u), kBufferFlags);
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) a_off[i] = ((uint32_t)min(m0 + srow + 32 * i, M - 1) * K + sch8) * 2u;
  const uint32_t w_thr = ((uint32_t)srow * K + sch8) * 2u;
  auto gload = [&](int i, int k0) -> u32x4 {
    if (i < A_CH)
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[i], k0 * 2, 0));
    const int j = i - A_CH;  // W rows 32 j .. 32 j + 31 of the tile
    int wr0;
    if (EPI == HL_EPI_SWIGLU)
      wr0 = (32 * j < BN / 2) ? nt * (BN / 2) + 32 * j : half_n + nt * (BN / 2) + 32 * j - BN / 2;
    else
      wr0 = nt * BN + 32 * j;
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, w_thr, (int)(((uint32_t)wr0 * K + (uint32_t)k0) * 2u), 0));
  };
  // 32 rows are 4096 bytes and keep the swizzle phase, so chunk i lands 4096 i past chunk 0
  const int dst0 = swz(srow, tid & 7);
  auto dst = [&](int i) { return i < A_CH ? dst0 + 4096 * i : C::A_BYTES + dst0 + 4096 * (i - A_CH); };
  // Fragments: a lane reads row lane % 16 of a 16-row block, 16-byte chunk 4 ks + lane / 16 (8
  // consecutive k) of step ks; A and W use the same k order, so the products sum the right terms.
  // A block i sits 2048 i past block 0 (16 rows keep the swizzle phase); W block t at
  // 128 * w_block_row(t).
  int fa_off[KS], fw_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    fa_off[ks] = swz(wm * C::WM + (lane & 15), 4 * ks + (lane >> 4));
    fw_off[ks] = C::A_BYTES + swz(lane & 15, 4 * ks + (lane >> 4));
  }
  int w_row[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) w_row[t] = 128 * w_block_row<EPI, BN, C::WN, NT>(wn, t);
  if constexpr (MC) {
    // cleared through the matrix core: with a plain zero store the split-K kernels' loops moved
    // every accumulator block to other registers once per k-step (the 256-wide one-tile loops
    // are clean either way and keep the plain store)
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[i][t] = mfma16x16x32(z, z, f32x4{});
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{};
  }

  // D = load depth: tile t + D - 1 is loaded while tile t is multiplied. D = 3 keeps two staging
  // register sets in flight (k-step t writes set (t - kb) % 2, which holds tile t + 1, to LDS and
  // refills it with tile t + 3), which gives a load two k-steps to arrive instead of one.
  static_assert(D == 2 || D == 3, "load depth");
  u32x4 rg[D - 1][NCH];
  u32x4 fa[MT], fw[2][NT];
  // fragment read j of a step: W block j (j < NT) into set `set`, else A block j - NT
  auto rd1 = [&](const uint8_t* base, int set, int ks, int j) {
    if (j < NT) fw[set][j] = *reinterpret_cast<const u32x4*>(base + fw_off[ks] + w_row[j]);
    else fa[j - NT] = *reinterpret_cast<const u32x4*>(base + fa_off[ks] + 2048 * (j - NT));
  };

  const int last = (ke - 1) * BK;
  // With two staging sets the loop runs k-steps in pairs; an odd count starts one step early on
  // a tile of zeros (A and W), which adds nothing to the sums. (A lone last step after the paired
  // loop, or a second loop for odd counts, makes the register allocator rotate the accumulators
  // inside the loop.)
  const int kf = D == 3 ? kb - ((ke - kb) & 1) : kb;
  if (kf < kb) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) rg[0][i] = u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i) rg[0][i] = gload(i, kb * BK);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(smem + dst(i)) = rg[0][i];
  // two sets are loaded one after the other, so the wait counts at the loop head are the steady
  // ones
#pragma unroll
  for (int s = 0; s < D - 1; ++s) {
    if constexpr (D == 3) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) rg[s][i] = gload(i, min((kf + 1 + s) * BK, last));
  }
  if constexpr (D == 3) __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NR; ++j) rd1(smem, 0, 0, j);

  // MFMA q of a step is (A block q / NT, W block q % NT). Fragment read j follows MFMA
  // (j + 1) NM / NR - 1, which for an A block j - NT is never before the step's last use of it;
  // staging pair i (step 0 only) follows MFMA i NM / NCH. Step 1 follows the barrier and reads
  // the next tile's step-0 fragments from the other buffer.
  auto kstep = [&](const int kt, u32x4 (&rgs)[NCH]) __attribute__((always_inline)) {
    const int buf = (kt - kf) & 1;
    const uint8_t* ab = smem + buf * C::STAGE;
    uint8_t* nb = smem + (buf ^ 1) * C::STAGE;
    const int knext = min((kt + D) * BK, last);  // past the end: re-read the last tile (unused)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks, nx = ks ^ 1;
      if (ks == KS - 1) {
        // tile t+1 complete in the other buffer; every read of this buffer has been issued
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* rbase = (ks == KS - 1) ? nb : ab;
      const int rks = (ks == KS - 1) ? 0 : ks + 1;
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        acc[q / NT][q % NT] = mfma16x16x32(fa[q / NT], fw[cur][q % NT], acc[q / NT][q % NT]);
        const int si = stage_after(q, NM, NCH), rj = read_after(q, NM, NR);
        if (ks == 0 && si >= 0) {
          *reinterpret_cast<u32x4*>(nb + dst(si)) = rgs[si];
          // keeps the write before the load that reuses its registers: without the pin the
          // register allocator splits the staging ranges and evicts an accumulator set
          __builtin_amdgcn_sched_barrier(0);
          rgs[si] = gload(si, knext);
        }
        if (rj >= 0) rd1(rbase, nx, rks, rj);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (D == 3) {
    for (int kt = kf; kt < ke; kt += 2) {
      kstep(kt, rg[0]);
      kstep(kt + 1, rg[1]);
    }
  } else {
    for (int kt = kb; kt < ke; ++kt) kstep(kt, rg[0]);
  }
  // the next call (stream-K) or the epilogue reuses the LDS
  __syncthreads();
}

// Reads an accumulator register inside the block that needs it. A plain use of the value by
// ordinary arithmetic lets the register allocator copy every accumulator out right after its
// last product, on the hot path, even when the consuming block rarely runs.
HL_DEV float agpr_read(float x) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
  return v;
}

// A stream-K run: iterations [it0, it1) of the (tile, k-step) sequence (tile j / nk, k-step
// j % nk, tiles numbered M-fastest) as one software pipeline that does not drain at tile
// boundaries. The staging, fragment and MFMA schedule per iteration is the one-tile loop's; the
// loads of iteration j + 2 take their tile's A rows and W rows. After the last k-step of a tile,
// or of the run, flush(tile, kb, ke, segment) consumes acc, which is then cleared.
template <int EPI, int BM, int BN, typename Flush>
HL_DEV void runloop(const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, int M, int N,
                    int K, int mtiles, int nk, int it0, int it1, uint8_t* smem,
                    f32x4 (&acc)[Cfg<BM, BN>::MT][Cfg<BM, BN>::NT], Flush&& flush) {
  using C = Cfg<BM, BN>;
  constexpr int MT = C::MT, NT = C::NT, NCH = C::NCH, A_CH = C::A_CH;
  constexpr int NM = MT * NT, NR = MT + NT, KS = BK / 32;
  static_assert(KS == 2, "the W fragment sets alternate per step and must line up across tiles");
  static_assert(EPI != HL_EPI_SWIGLU, "stream-K runs carry plain and residual GEMMs only");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int srow = tid >> 3, sch8 = (tid & 7) * 8;
  const __amdgpu_buffer_rsrc_t rs_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<hl_bf16*>(A), 0, (int)((uint32_t)M * (uint32_t)K * 2u), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_w =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<hl_bf16*>(W), 0, (int)((uint32_t)N * (uint32_t)K * 2u), kBufferFlags);
  const uint32_t w_thr = ((uint32_t)srow * K + sch8) * 2u;
  // source of iteration j: per-thread A row offsets, the tile's first W row, the k byte offset
  uint32_t a_off[A_CH];
  int w_row0 = 0, k_byte = 0;
  auto locate = [&](int j) {
    const int tile = j / nk, ks = j - tile * nk;
    const int mt = tile % mtiles, nt = tile / mtiles;
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      a_off[i] = ((uint32_t)min(mt * BM + srow + 32 * i, M - 1) * K + sch8) * 2u;
    w_row0 = nt * BN;
    k_byte = ks * BK * 2;
  };
  auto gload = [&](int i) -> u32x4 {
    if (i < A_CH)
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[i], k_byte, 0));
    const int wr0 = w_row0 + 32 * (i - A_CH);
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, w_thr, (int)((uint32_t)wr0 * K * 2u) + k_byte, 0));
  };
  const int dst0 = swz(srow, tid & 7);
  auto dst = [&](int i) { return i < A_CH ? dst0 + 4096 * i : C::A_BYTES + dst0 + 4096 * (i - A_CH); };
  int fa_off[KS], fw_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    fa_off[ks] = swz(wm * C::WM + (lane & 15), 4 * ks + (lane >> 4));
    fw_off[ks] = C::A_BYTES + swz(lane & 15, 4 * ks + (lane >> 4));
  }
  int w_row[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) w_row[t] = 128 * w_block_row<EPI, BN, C::WN, NT>(wn, t);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{};

  u32x4 rg[NCH];
  u32x4 fa[MT], fw[2][NT];
  auto rd1 = [&](const uint8_t* base, int set, int ks, int j) {
    if (j < NT) fw[set][j] = *reinterpret_cast<const u32x4*>(base + fw_off[ks] + w_row[j]);
    else fa[j - NT] = *reinterpret_cast<const u32x4*>(base + fa_off[ks] + 2048 * (j - NT));
  };

  locate(it0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) rg[i] = gload(i);
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(smem + dst(i)) = rg[i];
  locate(min(it0 + 1, it1 - 1));
#pragma unroll
  for (int i = 0; i < NCH; ++i) rg[i] = gload(i);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NR; ++j) rd1(smem, 0, 0, j);

  int seg = 0, seg_begin = it0;
  for (int cur = it0; cur < it1; ++cur) {
    const int buf = (cur - it0) & 1;
    const uint8_t* ab = smem + buf * C::STAGE;
    uint8_t* nb = smem + (buf ^ 1) * C::STAGE;
    locate(min(cur + 2, it1 - 1));  // past the end: re-read the last iteration (unused)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur_set = ks, nx = ks ^ 1;
      if (ks == KS - 1) {
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* rbase = (ks == KS - 1) ? nb : ab;
      const int rks = (ks == KS - 1) ? 0 : ks + 1;
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        acc[q / NT][q % NT] = mfma16x16x32(fa[q / NT], fw[cur_set][q % NT], acc[q / NT][q % NT]);
        const int si = stage_after(q, NM, NCH), rj = read_after(q, NM, NR);
        if (ks == 0 && si >= 0) {
          *reinterpret_cast<u32x4*>(nb + dst(si)) = rg[si];
          __builtin_amdgcn_sched_barrier(0);
          rg[si] = gload(si);
        }
        if (rj >= 0) rd1(rbase, nx, rks, rj);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int tile = cur / nk;
    if (cur + 1 == it1 || (cur + 1) % nk == 0) {
      flush(tile, seg_begin - tile * nk, cur + 1 - tile * nk, seg);
      // cleared through the matrix core: a plain zero store here makes the register allocator
      // shuttle every accumulator through ordinary registers inside the main loop
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma16x16x32(z, z, f32x4{});
      ++seg;
      seg_begin = cur + 1;
    }
  }
  __syncthreads();
}

// Row of the 16 x 16 output block held in accumulator register r of a lane: 4 (lane / 16) + r;
// its column is lane % 16.
HL_DEV int block_row(int lane, int r) { return (lane >> 4) * 4 + r; }

// RoPE + KV append for 8 pairs of one staged row: `srow` points at the fp32 row of one head.
// Only decode tokens (`decode`) get the low half of q: decode attention alone reads it.
template <int HD>
HL_DEV void rope_store_vals(const GemmEpi& ep, int gm, int gh, int blk, int slot, bool decode,
                            float (&a)[8], float (&b)[8], int c);

template <int HD>
HL_DEV void rope_store_row(const GemmEpi& ep, int gm, int gh, int blk, int slot, bool decode,
                           const float* srow, int c) {
  constexpr int half = HD / 2;
  float a[8], b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = srow[8 * c + e];
    b[e] = srow[half + 8 * c + e];
  }
  rope_store_vals<HD>(ep, gm, gh, blk, slot, decode, a, b, c);
}

// The same for values already in registers: a = elements 8c .. 8c+7 of the head, b = the
// elements d/2 apart from them (their rotation partners). q, k and v go out as non-temporal
// stores (store_nt): attention reads them next.
template <int HD>
HL_DEV void rope_store_vals(const GemmEpi& ep, int gm, int gh, int blk, int slot, bool decode,
                            float (&a)[8], float (&b)[8], int c) {
  constexpr int half = HD / 2;
  const int Hq = ep.n_q_heads, Hkv = ep.n_kv_heads;
  if (gh < Hq + Hkv) {
    const float2* cs = ep.rope_cs + (size_t)gm * half + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = cs[e];
      const float ra = a[e] * t.x - b[e] * t.y, rb = b[e] * t.x + a[e] * t.y;
      a[e] = ra;
      b[e] = rb;
    }
  }
  auto pack8 = [](const float* v) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
    return o;
  };
  if (gh < Hq) {
    const size_t o = ((size_t)gm * Hq + gh) * HD + 8 * c;
    store_nt(reinterpret_cast<u32x4*>(ep.q_rot + o), pack8(a));
    store_nt(reinterpret_cast<u32x4*>(ep.q_rot + o + half), pack8(b));
    if (ep.q_lo && decode) {  // what bf16 dropped, so decode attention can use q to ~16 bits
      float la[8], lb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        la[e] = a[e] - bf2f(f2bf(a[e]));
        lb[e] = b[e] - bf2f(f2bf(b[e]));
      }
      store_nt(reinterpret_cast<u32x4*>(ep.q_lo + o), pack8(la));
      store_nt(reinterpret_cast<u32x4*>(ep.q_lo + o + half), pack8(lb));
    }
    return;
  }
  if (blk < 0) return;
  if (gh < Hq + Hkv) {
    hl_bf16* page = ep.kpool + ((size_t)blk * Hkv + (gh - Hq)) * HL_BLOCK_SIZE * HD;
    store_nt(reinterpret_cast<u32x4*>(page + kpage_off(slot, c)), pack8(a));
    store_nt(reinterpret_cast<u32x4*>(page + kpage_off(slot, c + HD / 16)), pack8(b));
  } else {
    hl_bf16* dst = ep.vpool + ((size_t)blk * Hkv + (gh - Hq - Hkv)) * HD * HL_BLOCK_SIZE + slot;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      store_nt(dst + (size_t)(8 * c + e) * HL_BLOCK_SIZE, (hl_bf16)f2bf(a[e]));
      store_nt(dst + (size_t)(half + 8 * c + e) * HL_BLOCK_SIZE, (hl_bf16)f2bf(b[e]));
    }
  }
}

// The V rows of a staged fp32 tile into the Vᵀ pages. A page holds a head's values d-major
// ([d][16 slots]), so one token's row is 128 two-byte stores 32 bytes apart, and a store
// instruction costs one memory request per 32-byte piece it touches. Each lane stores 8 values of
// one row, and the lanes of one store go 16 rows by 4 adjacent d: when the 16 rows are
// consecutive tokens of one page (a prompt chunk), an instruction writes 4 whole 32-byte pieces;
// lanes along 8-element runs of one row (as for q and k) made 16 requests per instruction there.
// A decode row is alone in its page either way. `row_of(rr, blk, slot)`
// gives staged row rr's page and slot, false for a row past the end or without a page. Every
// thread of the workgroup calls it.
template <int HD, class RowOf>
HL_DEV void v_append_rows(const GemmEpi& ep, const float* st, int sstride, int rows, int gh_base,
                          int heads, RowOf row_of) {
  const int v0 = ep.n_q_heads + ep.n_kv_heads;  // first V head among the projection's columns
  const int h0 = max(v0 - gh_base, 0), h1 = min(heads, v0 + ep.n_kv_heads - gh_base);
  const int nvh = h1 - h0;
  if (nvh <= 0) return;
  const int groups = (rows + 15) / 16;
  constexpr int DG = HD / 8;  // runs of 8 d per lane; the lanes of a store cover 16 rows x 4 runs
  for (int e = threadIdx.x; e < groups * 16 * nvh * DG; e += blockDim.x) {
    const int rl = e & 15, dq = (e >> 4) & 3, rest = e >> 6;
    const int db = rest % (DG / 4), rest2 = rest / (DG / 4);
    const int hv = rest2 % nvh, rr = (rest2 / nvh) * 16 + rl;
    int blk, slot;
    if (rr >= rows || !row_of(rr, blk, slot)) continue;
    const int hi = h0 + hv;
    const float* src = st + rr * sstride + hi * HD;
    hl_bf16* dst = ep.vpool + ((size_t)blk * ep.n_kv_heads + (gh_base + hi - v0)) * HD * HL_BLOCK_SIZE + slot;
    // run j of the lane's 8 values: d = 32 db + 4 j + dq, so one instruction's 4 lanes of a row
    // take 4 adjacent d-rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 32 * db + 4 * j + dq;
      store_nt(dst + (size_t)d * HL_BLOCK_SIZE, (hl_bf16)f2bf(src[d]));
    }
  }
}

// The residual of one 16-row block row of a lane's accumulators (rows row0 + block_row(lane, r),
// columns col0 + 16 t + lane % 16), loaded before any of the row's stores and without branches: a
// load that follows a store to C in program order stays behind it (the two may alias), and a
// branch around a load waits for it before the paths join, so either costs one memory round trip
// per load. Rows past M read row M - 1 (never stored). Raw bf16 bits; the caller converts.
template <int NT>
HL_DEV void load_residual_row(const GemmEpi& ep, uint32_t (&res)[4][NT], int row0, int col0,
                              int M, int N, int lane) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const hl_bf16* p =
        ep.residual + (size_t)min(row0 + block_row(lane, r), M - 1) * N + col0 + (lane & 15);
#pragma unroll
    for (int t = 0; t < NT; ++t) res[r][t] = p[t * 16];
  }
}

// SK: stream-K run of (tile, k-step) iterations; otherwise exactly one tile per workgroup (kept a
// separate instantiation so the one-tile kernels carry no loop state in registers).
template <int EPI, int BM, int BN, int HD, bool SK>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_nt_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, hl_bf16* __restrict__ C, int M,
    int N, int K, GemmEpi ep, Sched sc) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float rs_sh[BM];
  __shared__ int pos_sh[BM];
  __shared__ int blk_sh[BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lc = lane & 15;
  const int half_n = N >> 1;
  const int tiles = sc.mtiles * sc.ntiles;

  // work: one tile, or a stream-K run of (tile, k-step) iterations. Runs are normally
  // XCD-contiguous (the runs of one XCD cover adjacent tiles, the M tiles of one or two N columns,
  // whose operands its L2 can hold for short K); with phase_runs, run r goes to XCD r mod 8, which
  // puts runs that start at the same k-step on the same M tile of successive N columns together
  // (they read the same A slices at the same time; for long K nothing else would be reused).
  const int run = (SK && sc.phase_runs) ? (int)blockIdx.x : xcd_tile(blockIdx.x, gridDim.x);
  int it = 0, it_end = 0;
  if constexpr (!SK) {
    it = run * sc.nk;
    it_end = it + sc.nk;
  } else {
    it = run * sc.ipw;
    it_end = min(it + sc.ipw, tiles * sc.nk);
  }
  if constexpr (SK) {
    // Stream-K (plain / residual epilogues): pieces of split tiles go to the workspace for the
    // fix-up kernel (slot 0 = the first segment of this run, slot 1 = its last), in register
    // order: block (i, t) of wave w is 64 lanes x 4 floats at ((w MT + i) NT + t) 256, one 1 KB
    // store per block. Tiles whole in this run are finished here.
    f32x4 acc[MT][NT];
    runloop<EPI, BM, BN>(A, W, M, N, K, sc.mtiles, sc.nk, it, it_end, smem, acc,
                         [&](int tile, int kb, int ke, int seg) {
      // The flush runs inside the pipelined loop: the thread index is passed through an opaque
      // move so that none of the epilogue's per-lane address arithmetic is hoisted out of the
      // loop (where it would occupy registers the main loop needs).
      int tid2;
      asm volatile("v_mov_b32 %0, %1" : "=v"(tid2) : "v"(tid));
      const int lane = tid2 & 63, lc = lane & 15;
      const int wave = __builtin_amdgcn_readfirstlane(tid2 >> 6), wm = wave >> 1, wn = wave & 1;
      if (kb != 0 || ke != sc.nk) {
        float* pdst = sc.part + ((size_t)run * 2 + (seg == 0 ? 0 : 1)) * BM * BN;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4*>(pdst + ((wave * MT + i) * NT + t) * 256 + lane * 4) = acc[i][t];
        return;
      }
      const int m0 = (tile % sc.mtiles) * BM, nt = tile / sc.mtiles;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        uint32_t res[4][NT];
        if constexpr (EPI == HL_EPI_RESIDUAL)
          load_residual_row<NT>(ep, res, m0 + wm * CF::WM + i * 16, nt * BN + wn * CF::WN, M, N,
                                lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gm = m0 + wm * CF::WM + i * 16 + block_row(lane, r);
          if (gm >= M) continue;
          const float rs = ep.row_scale ? ep.row_scale[gm] : 1.f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const size_t o = (size_t)gm * N + nt * BN + wn * CF::WN + t * 16 + lc;
            float v = agpr_read(acc[i][t][r]) * rs;
            if constexpr (EPI == HL_EPI_RESIDUAL) v += bf2f(res[r][t]);
            C[o] = (hl_bf16)f2bf(v);
          }
        }
      }
    });
    return;
  } else {
    const int tile = it / sc.nk;
    const int mt = tile % sc.mtiles, nt = tile / sc.mtiles;
    const int m0 = mt * BM;
    f32x4 acc[MT][NT];
    mainloop<EPI, BM, BN>(A, W, M, N, K, mt, nt, 0, sc.nk, smem, acc);
    if (tid < BM) {
      const int gm = m0 + tid;
      rs_sh[tid] = (ep.row_scale && gm < M) ? ep.row_scale[gm] : 1.f;
      if (EPI == kEpiRopeAppend) {
        pos_sh[tid] = gm < M ? ep.tok_pos[gm] : 0;
        blk_sh[tid] = gm < M ? ep.tok_blk[gm] : -1;
      }
    }
    __syncthreads();
    if constexpr (EPI == HL_EPI_SWIGLU) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * CF::WM + i * 16 + block_row(lane, r), gm = m0 + row;
          if (gm >= M) continue;
          const float rs = rs_sh[row];
#pragma unroll
          for (int t = 0; t < NT / 2; ++t) {
            const float g = acc[i][t][r] * rs, u = acc[i][t + NT / 2][r] * rs;
            C[(size_t)gm * half_n + nt * (BN / 2) + wn * (CF::WN / 2) + t * 16 + lc] =
                (hl_bf16)f2bf(silu(g) * u);
          }
        }
    } else if constexpr (EPI == kEpiRopeAppend) {
      // stage the scaled fp32 tile in LDS, then rotate / route whole 8-element runs; a 256-row
      // tile is staged one wave row (128 rows) at a time so the stage fits in the main-loop LDS
      constexpr int NPASS = BM > 128 ? 2 : 1, PROWS = BM / NPASS;
      float* st = reinterpret_cast<float*>(smem);
      constexpr int SROW = kStageRow<BN>;  // padded: the 4 row groups of a store hit distinct banks
      constexpr int heads = BN / HD, chunks = HD / 16;
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        if (NPASS == 1 || wm == pass) {
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = wm * CF::WM + i * 16 + block_row(lane, r);
#pragma unroll
              for (int t = 0; t < NT; ++t)
                st[(row - pass * PROWS) * SROW + wn * CF::WN + t * 16 + lc] = acc[i][t][r] * rs_sh[row];
            }
        }
        __syncthreads();
        const int vfirst = ep.n_q_heads + ep.n_kv_heads;  // q and k heads here, V heads below
        for (int e = tid; e < PROWS * heads * chunks; e += kThreads) {
          const int c = e % chunks, rest = e / chunks, hi = rest % heads, rr = rest / heads;
          const int r = pass * PROWS + rr, gm = m0 + r;
          if (gm >= M || nt * heads + hi >= vfirst) continue;
          rope_store_row<HD>(ep, gm, nt * heads + hi, blk_sh[r], pos_sh[r] & (HL_BLOCK_SIZE - 1),
                             (pos_sh[r] & hl::kDecodeBit) != 0, st + rr * SROW + hi * HD, c);
        }
        v_append_rows<HD>(ep, st, SROW, PROWS, nt * heads, heads, [&](int rr, int& blk, int& slot) {
          const int r = pass * PROWS + rr;
          blk = blk_sh[r];
          slot = pos_sh[r] & (HL_BLOCK_SIZE - 1);
          return m0 + r < M && blk >= 0;
        });
        if (NPASS > 1) __syncthreads();
      }
    } else {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        uint32_t res[4][NT];
        if constexpr (EPI == HL_EPI_RESIDUAL)
          load_residual_row<NT>(ep, res, m0 + wm * CF::WM + i * 16, nt * BN + wn * CF::WN, M, N,
                                lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * CF::WM + i * 16 + block_row(lane, r), gm = m0 + row;
          if (gm >= M) continue;
          const float rs = rs_sh[row];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const size_t o = (size_t)gm * N + nt * BN + wn * CF::WN + t * 16 + lc;
            float v = acc[i][t][r] * rs;
            if constexpr (EPI == HL_EPI_RESIDUAL) v += bf2f(res[r][t]);
            C[o] = (hl_bf16)f2bf(v);
          }
        }
      }
    }
  }
}

// Stream-K fix-up: for each split tile, sum its pieces and apply the plain or residual epilogue
// (stream-K is used only for those). Pieces are in the main kernel's register order; a thread
// takes lanes 4 q .. 4 q + 3 of one 16 x 16 block (16 consecutive floats of each piece), which are
// 4 consecutive columns of 4 rows, so every output row gets one 8-byte store.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(hl_bf16* __restrict__ C, int M, int N,
                                                         GemmEpi ep, Sched sc) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT;
  const int tile = blockIdx.x;
  const int first = tile * sc.nk, lastit = first + sc.nk - 1;
  const int w0 = first / sc.ipw, w1 = lastit / sc.ipw;
  if (w0 == w1) return;  // finished in one piece by the main kernel
  const int mt = tile % sc.mtiles, nt = tile / sc.mtiles;
  const int g = blockIdx.y * 256 + threadIdx.x;  // quad index within the tile
  const int q = g & 15, blk = g >> 4;            // lane quad, block (w MT + i) NT + t
  const int t = blk % NT, i = (blk / NT) % MT, w = blk / (NT * MT);
  const int row0 = (w >> 1) * CF::WM + i * 16 + (q >> 2) * 4;
  const int col = (w & 1) * CF::WN + t * 16 + (q & 3) * 4;
  f32x4 v[4] = {};  // v[l][r]: column col + l, row row0 + r
  // piece of run wg (slot 0 if the tile is the first segment of wg's run)
  auto piece = [&](int wg) {
    const int slot = ((wg * sc.ipw) / sc.nk == tile) ? 0 : 1;
    return reinterpret_cast<const f32x4*>(sc.part + ((size_t)wg * 2 + slot) * BM * BN + blk * 256 +
                                          q * 16);
  };
  // a short K split over many runs leaves a tile in many pieces: four pieces' loads are issued
  // together, then added in run order
  int wg = w0;
  for (; wg + 3 <= w1; wg += 4) {
    f32x4 t[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4* src = piece(wg + u);
#pragma unroll
      for (int l = 0; l < 4; ++l) t[u][l] = src[l];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int l = 0; l < 4; ++l) v[l] += t[u][l];
  }
  for (; wg <= w1; ++wg) {
    const f32x4* src = piece(wg);
#pragma unroll
    for (int l = 0; l < 4; ++l) v[l] += src[l];
  }
  // the residual rows and row scales, loaded before any store (see load_residual_row)
  u32x2 rres[4];
  float rsv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = min(mt * BM + row0 + r, M - 1);
    rres[r] = ep.kind == HL_EPI_RESIDUAL
                  ? *reinterpret_cast<const u32x2*>(ep.residual + (size_t)gm * N + nt * BN + col)
                  : u32x2{0u, 0u};
    rsv[r] = ep.row_scale ? ep.row_scale[gm] : 1.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = mt * BM + row0 + r;
    if (gm >= M) break;
    const size_t o = (size_t)gm * N + nt * BN + col;
    const float rs = rsv[r];
    float e[4] = {v[0][r] * rs, v[1][r] * rs, v[2][r] * rs, v[3][r] * rs};
    if (ep.kind == HL_EPI_RESIDUAL) {
      const u32x2 rr = rres[r];
      e[0] += bf_lo(rr[0]);
      e[1] += bf_hi(rr[0]);
      e[2] += bf_lo(rr[1]);
      e[3] += bf_hi(rr[1]);
    }
    *reinterpret_cast<u32x2*>(C + o) = u32x2{pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3])};
  }
}

// Split-K main kernel: workgroup (tile, s) runs k-steps [s nk / S, (s + 1) nk / S) of its tile
// and stores the fp32 accumulators in register order as piece (s, tile): block (i, t) of wave w
// is 64 lanes x 4 floats at ((w MT + i) NT + t) 256. Workgroups are numbered tile-fastest per
// split and dealt XCD-contiguously, so the M tiles of one weight column run together.
template <int EPI, int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_split_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, int M, int N, int K,
    int splits, int mtiles, int tiles, float* __restrict__ part, int tile0) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // `tiles` tiles from tile tile0 of the GEMM on; pieces are numbered from 0
  const int u = xcd_tile(blockIdx.x, gridDim.x);
  const int tile = u % tiles, s = u / tiles, gt = tile0 + tile;
  const int nk = K / BK;
  const int kb = (int)((long)s * nk / splits), ke = (int)((long)(s + 1) * nk / splits);
  f32x4 acc[MT][NT];
  mainloop<EPI, BM, BN, 2, true>(A, W, M, N, K, gt % mtiles, gt / mtiles, kb, ke, smem, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* dst = part + ((size_t)s * tiles + tile) * BM * BN + lane * 4;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<f32x4*>(dst + ((wave * MT + i) * NT + t) * 256) = acc[i][t];
}

// Split-K fix-up, plain / residual: a thread takes one lane quad (4 columns x 4 rows) of one
// 16 x 16 block, sums its S pieces in split order and applies the epilogue.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_split_fixup(hl_bf16* __restrict__ C, int M, int N,
                                                        GemmEpi ep, int splits, int mtiles,
                                                        int tiles, const float* __restrict__ part,
                                                        int tile0) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT;
  // pieces of `tiles` split tiles, the first of which is tile tile0 of the GEMM
  const int tile = blockIdx.x, mt = (tile0 + tile) % mtiles, nt = (tile0 + tile) / mtiles;
  const int g = blockIdx.y * 256 + threadIdx.x;
  const int q = g & 15, blk = g >> 4;  // lane quad, block (w MT + i) NT + t
  if (blk >= 4 * MT * NT) return;
  const int t = blk % NT, i = (blk / NT) % MT, w = blk / (NT * MT);
  f32x4 v[4] = {};
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(part + ((size_t)s * tiles + tile) * BM * BN +
                                                      blk * 256 + q * 16);
#pragma unroll
    for (int l = 0; l < 4; ++l) v[l] += src[l];
  }
  const int row0 = mt * BM + (w >> 1) * CF::WM + i * 16 + (q >> 2) * 4;
  const int col = nt * BN + (w & 1) * CF::WN + t * 16 + (q & 3) * 4;
  // the residual rows and row scales, loaded before any store (see load_residual_row)
  u32x2 rres[4];
  float rsv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = min(row0 + r, M - 1);
    rres[r] = ep.kind == HL_EPI_RESIDUAL
                  ? *reinterpret_cast<const u32x2*>(ep.residual + (size_t)gm * N + col)
                  : u32x2{0u, 0u};
    rsv[r] = ep.row_scale ? ep.row_scale[gm] : 1.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = row0 + r;
    if (gm >= M) break;
    const size_t o = (size_t)gm * N + col;
    const float rs = rsv[r];
    float e[4] = {v[0][r] * rs, v[1][r] * rs, v[2][r] * rs, v[3][r] * rs};
    if (ep.kind == HL_EPI_RESIDUAL) {
      const u32x2 rr = rres[r];
      e[0] += bf_lo(rr[0]);
      e[1] += bf_hi(rr[0]);
      e[2] += bf_lo(rr[1]);
      e[3] += bf_hi(rr[1]);
    }
    *reinterpret_cast<u32x2*>(C + o) = u32x2{pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3])};
  }
}

// Split-K fix-up, SwiGLU: a thread takes one lane quad (4 columns x 4 rows) of a gate block and
// the same quad of its up block (NT / 2 blocks later in the same wave), sums the S pieces of
// each in split order, and writes silu(gate) * up.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_split_swiglu_fixup(hl_bf16* __restrict__ C, int M,
                                                               int N, GemmEpi ep, int splits,
                                                               int mtiles, int tiles,
                                                               const float* __restrict__ part,
                                                               int tile0) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT, NH = NT / 2;
  const int tile = blockIdx.x, mt = (tile0 + tile) % mtiles, nt = (tile0 + tile) / mtiles;
  const int g = blockIdx.y * 256 + threadIdx.x;
  const int q = g & 15, hb = g >> 4;  // lane quad, gate block (w, i, t < NH)
  if (hb >= 4 * MT * NH) return;
  const int t = hb % NH, i = (hb / NH) % MT, w = hb / (NH * MT);
  const int bg = (w * MT + i) * NT + t, bu = bg + NH;
  f32x4 vg[4] = {}, vu[4] = {};
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float* src = part + ((size_t)s * tiles + tile) * BM * BN + q * 16;
    const f32x4* pg = reinterpret_cast<const f32x4*>(src + bg * 256);
    const f32x4* pu = reinterpret_cast<const f32x4*>(src + bu * 256);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      vg[l] += pg[l];
      vu[l] += pu[l];
    }
  }
  const int half_n = N >> 1;
  const int row0 = mt * BM + (w >> 1) * CF::WM + i * 16 + (q >> 2) * 4;
  const int col = nt * (BN / 2) + (w & 1) * (CF::WN / 2) + t * 16 + (q & 3) * 4;
  float rsv[4];  // row scales loaded before any store (see load_residual_row)
#pragma unroll
  for (int r = 0; r < 4; ++r) rsv[r] = ep.row_scale ? ep.row_scale[min(row0 + r, M - 1)] : 1.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = row0 + r;
    if (gm >= M) break;
    const float rs = rsv[r];
    float e[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) e[l] = silu(vg[l][r] * rs) * (vu[l][r] * rs);
    *reinterpret_cast<u32x2*>(C + (size_t)gm * half_n + col) =
        u32x2{pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3])};
  }
}

// Split-K fix-up, RoPE + KV append: a workgroup takes 32 rows of a tile, sums the S pieces of
// each quad into an fp32 LDS stage (row-scaled), then rotates and routes whole 8-element runs of
// each head exactly as the one-tile epilogue does.
template <int BM, int BN, int HD>
__global__ __launch_bounds__(256) void gemm_split_rope_fixup(int M, GemmEpi ep, int splits,
                                                             int mtiles, int tiles,
                                                             const float* __restrict__ part,
                                                             int tile0) {
  using CF = Cfg<BM, BN>;
  constexpr int MT = CF::MT, NT = CF::NT, SROW = kStageRow<BN>, ROWS = 32;
  constexpr int CB = BN / 16;  // 16-column blocks of the tile
  __shared__ float st[ROWS * SROW];
  const int tile = blockIdx.x, mt = (tile0 + tile) % mtiles, nt = (tile0 + tile) / mtiles;
  const int r0 = blockIdx.y * ROWS;
  const int tid = threadIdx.x;
  for (int e = tid; e < (ROWS / 16) * CB * 16; e += 256) {
    const int q = e & 15, cb = (e >> 4) % CB, rb = (e >> 4) / CB;
    const int R = r0 / 16 + rb;  // 16-row block of the tile
    const int blk = (((R / MT) * 2 + cb / NT) * MT + R % MT) * NT + cb % NT;
    f32x4 v[4] = {};
#pragma unroll 4
    for (int s = 0; s < splits; ++s) {
      const f32x4* src =
          reinterpret_cast<const f32x4*>(part + ((size_t)s * tiles + tile) * BM * BN + blk * 256 + q * 16);
#pragma unroll
      for (int l = 0; l < 4; ++l) v[l] += src[l];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = rb * 16 + (q >> 2) * 4 + r, gm = mt * BM + r0 + rr;
      const float rs = (ep.row_scale && gm < M) ? ep.row_scale[gm] : 1.f;
#pragma unroll
      for (int l = 0; l < 4; ++l) st[rr * SROW + cb * 16 + (q & 3) * 4 + l] = v[l][r] * rs;
    }
  }
  __syncthreads();
  constexpr int heads = BN / HD, chunks = HD / 16;
  const int vfirst = ep.n_q_heads + ep.n_kv_heads;  // q and k heads here, V heads below
  for (int e = tid; e < ROWS * heads * chunks; e += 256) {
    const int c = e % chunks, rest = e / chunks, hi = rest % heads, rr = rest / heads;
    const int gm = mt * BM + r0 + rr;
    if (gm >= M || nt * heads + hi >= vfirst) continue;
    const int pos = ep.tok_pos[gm];
    rope_store_row<HD>(ep, gm, nt * heads + hi, ep.tok_blk[gm], pos & (HL_BLOCK_SIZE - 1),
                       (pos & hl::kDecodeBit) != 0, st + rr * SROW + hi * HD, c);
  }
  v_append_rows<HD>(ep, st, SROW, ROWS, nt * heads, heads, [&](int rr, int& blk, int& slot) {
    const int gm = mt * BM + r0 + rr;
    if (gm >= M) return false;
    blk = ep.tok_blk[gm];
    slot = ep.tok_pos[gm] & (HL_BLOCK_SIZE - 1);
    return blk >= 0;
  });
}

// Pieces of a split-K launch must fit the stream-K workspace.
inline bool split_fits(int m, int n, int bm, int bn, int splits) {
  const size_t tiles = (size_t)((m + bm - 1) / bm) * (n / bn);
  return (size_t)splits * tiles * bm * bn * 4 <= kStreamKWorkspace;
}
// Tail split: the tiles that run whole (the full rounds over the compute units), and whether
// the pieces of the rest fit the workspace.
inline int tail_full_tiles(int tiles) { return (tiles / kStreamKGrid) * kStreamKGrid; }
inline bool tail_fits(int tail, int bm, int bn, int splits) {
  return (size_t)splits * tail * bm * bn * 4 <= kStreamKWorkspace;
}

// The fix-up of `tiles` split tiles (the first is tile tile0 of the GEMM), `splits` pieces each.
template <int EPI, int BM, int BN, int HD>
hipError_t launch_split_fixup(hl_bf16* c, int m, int n, const GemmEpi& epi, const float* part,
                              int splits, int mtiles, int tiles, int tile0, hipStream_t st) {
  using CF = Cfg<BM, BN>;
  if constexpr (EPI == HL_EPI_SWIGLU) {
    constexpr int quads = 4 * CF::MT * (CF::NT / 2) * 16;
    hipLaunchKernelGGL((gemm_split_swiglu_fixup<BM, BN>), dim3(tiles, (quads + 255) / 256),
                       dim3(256), 0, st, c, m, n, epi, splits, mtiles, tiles, part, tile0);
  } else if constexpr (EPI == HL_EPI_NONE || EPI == HL_EPI_RESIDUAL) {
    constexpr int quads = 4 * CF::MT * CF::NT * 16;
    hipLaunchKernelGGL((gemm_split_fixup<BM, BN>), dim3(tiles, (quads + 255) / 256), dim3(256), 0,
                       st, c, m, n, epi, splits, mtiles, tiles, part, tile0);
  } else {
    hipLaunchKernelGGL((gemm_split_rope_fixup<BM, BN, HD>), dim3(tiles, BM / 32), dim3(256), 0,
                       st, m, epi, splits, mtiles, tiles, part, tile0);
  }
  return hipGetLastError();
}

// Split-K over all tiles, or (tail) over the tiles past the last full round only: those the
// one-tile launch before it left out.
template <int EPI, int BM, int BN, int HD>
hipError_t launch_split(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, float* part, int splits, hipStream_t st,
                        bool tail = false) {
  using CF = Cfg<BM, BN>;

  auto kern = gemm_split_kernel<EPI, BM, BN>;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, CF::MAIN_LDS);
    (void)hipGetLastError();
    attr = true;
  }
  const int mtiles = (m + BM - 1) / BM, tiles = mtiles * (n / BN);
  const int t0 = tail ? tail_full_tiles(tiles) : 0;
  hipLaunchKernelGGL(kern, dim3((tiles - t0) * splits), dim3(kThreads), CF::MAIN_LDS, st, a, w, m,
                     n, k, splits, mtiles, tiles - t0, part, t0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_split_fixup<EPI, BM, BN, HD>(c, m, n, epi, part, splits, mtiles, tiles - t0, t0,
                                             st);
}

template <int EPI, int BM, int BN, int HD = 0>
hipError_t launch_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, float* part, bool streamk, hipStream_t st,
                        int tail_splits = 0) {
  using CF = Cfg<BM, BN>;
  constexpr bool kCanSplit = (EPI == HL_EPI_NONE || EPI == HL_EPI_RESIDUAL);
  auto kern = gemm_bf16_nt_kernel<EPI, BM, BN, HD, false>;
  auto kern_sk = gemm_bf16_nt_kernel<EPI, BM, BN, HD, kCanSplit>;
  const int lds = (EPI == kEpiRopeAppend) ? max(CF::MAIN_LDS, min(BM, 128) * kStageRow<BN> * 4) : CF::MAIN_LDS;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern_sk),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipGetLastError();
    attr = true;
  }
  Sched sc;
  sc.mtiles = (m + BM - 1) / BM;
  sc.ntiles = n / BN;
  sc.nk = k / BK;
  sc.ipw = 0;
  sc.phase_runs = 0;
  sc.part = part;
  const int tiles = sc.mtiles * sc.ntiles;
  int grid = tiles;
  streamk = streamk && kCanSplit && part;
  // Tail split: the full rounds of tiles here, then the tiles left over (whose round would leave
  // most compute units idle) as split-K pieces in a launch of their own, which starts as the
  // equal-length tiles of the last full round drain together.
  bool tail = false;
  if (!streamk && part && tail_splits >= 2) {
    const int full = tail_full_tiles(tiles);
    tail = full < tiles && tail_fits(tiles - full, BM, BN, tail_splits) && tail_splits <= sc.nk;
    if (tail) grid = full;
  }
  if (streamk) {
    const int total = tiles * sc.nk;
    sc.ipw = (total + kStreamKGrid - 1) / kStreamKGrid;
    grid = (total + sc.ipw - 1) / sc.ipw;
    // runs r and r + period start at the same k-step, `adv` tiles apart; dispatch order puts
    // them on one XCD when the period is a multiple of 8, and on one M tile when adv is a
    // multiple of the M tile count (tiles are numbered M-fastest)
    int g = sc.ipw, h = sc.nk;
    while (h) { const int t = g % h; g = h; h = t; }
    const long period = sc.nk / g, adv = (long)sc.ipw * period / sc.nk;
    sc.phase_runs = (k >= 8192 && period % 8 == 0 && adv % sc.mtiles == 0) ? 1 : 0;
  }
  if (streamk)
    hipLaunchKernelGGL(kern_sk, dim3(grid), dim3(kThreads), lds, st, a, w, c, m, n, k, epi, sc);
  else if (grid > 0)
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, st, a, w, c, m, n, k, epi, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (BN == 192) {
    return e;  // the 192-wide SwiGLU tiles run one tile per workgroup only
  } else {
    if (tail) return launch_split<EPI, BM, BN, HD>(a, w, c, m, n, k, epi, part, tail_splits, st, true);
    if (!streamk) return e;
    hipLaunchKernelGGL((gemm_fixup_kernel<BM, BN>), dim3(tiles, BM * BN / 4096), dim3(256), 0, st,
                       c, m, n, epi, sc);
    return hipGetLastError();
  }
}

// Launch with the chosen tile shape: every shape below is compiled for the epilogue EPI.
template <int EPI, int HD = 0>
hipError_t launch_choice(const hl::TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                         int m, int n, int k, const GemmEpi& epi, float* part, hipStream_t st) {
  const bool sk = tc.sk && part != nullptr;
  const int ts = tc.tail ? tc.splits : 0;
  {
    if (tc.splits >= 2 && !tc.tail) {
      if (!part || !split_fits(m, n, tc.bm, tc.bn, tc.splits) || tc.splits > k / BK)
        return hipErrorInvalidValue;
      switch (tc.bm * 1000 + tc.bn) {
        case 256256: return launch_split<EPI, 256, 256, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 224256: return launch_split<EPI, 224, 256, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 192256: return launch_split<EPI, 192, 256, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 160256: return launch_split<EPI, 160, 256, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 128256: return launch_split<EPI, 128, 256, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 256128: return launch_split<EPI, 256, 128, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 224128: return launch_split<EPI, 224, 128, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 160128: return launch_split<EPI, 160, 128, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        case 128128: return launch_split<EPI, 128, 128, HD>(a, w, c, m, n, k, epi, part, tc.splits, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (tc.bm * 1000 + tc.bn) {
    case 256256: return launch_tiles<EPI, 256, 256, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 224256: return launch_tiles<EPI, 224, 256, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 192256: return launch_tiles<EPI, 192, 256, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 160256: return launch_tiles<EPI, 160, 256, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 128256: return launch_tiles<EPI, 128, 256, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 256128: return launch_tiles<EPI, 256, 128, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 224128: return launch_tiles<EPI, 224, 128, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 160128: return launch_tiles<EPI, 160, 128, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 128128: return launch_tiles<EPI, 128, 128, HD>(a, w, c, m, n, k, epi, part, sk, st, ts);
    case 256192:
    case 128192:
      // SwiGLU only, one tile per workgroup: 96 gate + 96 up rows per tile, so that 512 and 256
      // rows of a 2 x 12288-wide gate/up projection make exactly 256 tiles
      if constexpr (EPI == HL_EPI_SWIGLU) {
        if (sk || ts) return hipErrorInvalidValue;
        return tc.bm == 256 ? launch_tiles<EPI, 256, 192, HD>(a, w, c, m, n, k, epi, part, false, st)
                            : launch_tiles<EPI, 128, 192, HD>(a, w, c, m, n, k, epi, part, false, st);
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
