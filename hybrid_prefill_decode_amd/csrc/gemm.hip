// Token-batched linear layer on the CDNA4 matrix cores: C = A W^T (bf16 in, fp32 accumulate).
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?").
//
// Main loop (256 threads = 4 waves, one per SIMD; K advances 64 per tile). Each wave owns a
// (BM/2) x (BN/2) block of v_mfma_f32_32x32x16_bf16 outputs whose fp32 accumulators live in the
// accumulation registers (256 of them for a 256 x 256 tile), so the 256 ordinary registers stay
// free for fragments and staging. A and W tiles are staged through LDS in 128-byte rows whose
// 16-byte chunks are XOR-swizzled with (row / 2) mod 8, which keeps every 16-lane group of a
// fragment read on distinct banks. Per tile: k16 steps 0..2 each carry the fragment reads of
// the next step and a third of the tile's staging work (LDS writes of tile t+1 from registers,
// global loads of tile t+2 into them), issued one per MFMA in an order pinned with sched_barrier;
// the barrier sits before step 3, whose MFMAs hide the fragment reads of the next tile's step 0.
// Tiles are dealt so that consecutive tile ids land on the same XCD (workgroups go to the 8 XCDs
// round-robin) and, within an XCD, the M tiles of one N column run together, so a weight tile is
// fetched from HBM once.
//
// Schedules. Wide GEMMs run one tile per workgroup. Narrow ones (N = hidden for the O and down
// projections leaves fewer tiles than compute units) run stream-K: exactly one workgroup per CU,
// each taking an equal run of (tile, k-step) iterations; a tile split between workgroups is written
// as fp32 pieces to the workspace and finished by a fix-up kernel that sums the pieces and applies
// the epilogue.
//
// Epilogues, after an optional per-row scale (the RMSNorm factor, see prep.hip): plain, + residual,
// SwiGLU (the W tile holds BN/2 gate rows and the matching BN/2 up rows; a lane holds a gate and
// its up in registers), and RoPE + KV append for the QKV projection (the fp32 tile is staged in
// LDS; q heads are rotated into q_rot, k heads rotated and v heads copied into their cache pages).
#include "common.h"

namespace {
using hl::GemmEpi;
using hl::kEpiRopeAppend;

constexpr int BK = 64, kThreads = 256;
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
  static constexpr int MT = WM / 32, NT = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int A_CH = A_BYTES / 16 / kThreads, W_CH = W_BYTES / 16 / kThreads;
  static constexpr int NCH = A_CH + W_CH;
  static constexpr int PER = (NCH + 2) / 3;  // staging chunks per k16 step 0..2
  static constexpr int MAIN_LDS = 2 * STAGE;
  static_assert(A_CH * kThreads * 16 == A_BYTES && W_CH * kThreads * 16 == W_BYTES, "staging");
};

// Row of the W tile that feeds block t of wave column wn (SwiGLU pairs gate block t with up
// block t + NT/2 so both land in the same lane).
template <int EPI, int BN, int WN, int NT>
HL_DEV int w_block_row(int wn, int t) {
  if (EPI == HL_EPI_SWIGLU)
    return (t < NT / 2) ? wn * (WN / 2) + t * 32 : BN / 2 + wn * (WN / 2) + (t - NT / 2) * 32;
  return wn * WN + t * 32;
}

// One tile's K range [kb, ke) into acc (acc zeroed here).
template <int EPI, int BM, int BN>
HL_DEV void mainloop(const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, int M, int N,
                     int K, int mt, int nt, int kb, int ke, uint8_t* smem,
                     f32x16 (&acc)[Cfg<BM, BN>::MT][Cfg<BM, BN>::NT]) {
  using C = Cfg<BM, BN>;
  constexpr int MT = C::MT, NT = C::NT, NCH = C::NCH, A_CH = C::A_CH, PER = C::PER;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = mt * BM;
  const int half_n = N >> 1;

  // Staging: chunk i of a thread is row (tid / 8) + 32 i of the A tile (i < A_CH) or of the W
  // tile, 16-byte column tid % 8. Rows past M read row M-1: a C row depends only on its own A
  // row and padded C rows are never stored, so the loads need no branch. Offsets are 32-bit
  // element counts (the host bounds M K and N K below 2^31); the W row bases are wave-uniform.
  const int srow = tid >> 3, sch8 = (tid & 7) * 8;
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) a_off[i] = (uint32_t)min(m0 + srow + 32 * i, M - 1) * K + sch8;
  const uint32_t w_thr = (uint32_t)srow * K + sch8;
  auto gsrc = [&](int i, int k0) {
    if (i < A_CH) return reinterpret_cast<const u32x4*>(A + (a_off[i] + (uint32_t)k0));
    const int j = i - A_CH;  // W rows 32 j .. 32 j + 31 of the tile
    int wr0;
    if (EPI == HL_EPI_SWIGLU)
      wr0 = (32 * j < BN / 2) ? nt * (BN / 2) + 32 * j : half_n + nt * (BN / 2) + 32 * j - BN / 2;
    else
      wr0 = nt * BN + 32 * j;
    return reinterpret_cast<const u32x4*>(W + ((uint32_t)wr0 * K + w_thr + (uint32_t)k0));
  };
  // 32 rows are 4096 bytes and keep the swizzle phase, so chunk i lands 4096 i past chunk 0
  const int dst0 = swz(srow, tid & 7);
  auto dst = [&](int i) { return i < A_CH ? dst0 + 4096 * i : C::A_BYTES + dst0 + 4096 * (i - A_CH); };
  // fragment offsets per k16 step: A block i at + 4096 i, W block t at + 128 * w_block_row(t)
  int fa_off[BK / 16], fw_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    fa_off[ks] = swz(wm * C::WM + (lane & 31), 2 * ks + (lane >> 5));
    fw_off[ks] = C::A_BYTES + swz(lane & 31, 2 * ks + (lane >> 5));
  }
  int w_row[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) w_row[t] = 128 * w_block_row<EPI, BN, C::WN, NT>(wn, t);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x16{};

  u32x4 rg[NCH];
  u32x4 fa[2][MT], fw[2][NT];
  // fragment q of a step: A block q (q < MT) or W block q - MT
  auto rd1 = [&](const uint8_t* base, int set, int ks, int q) {
    if (q < MT) fa[set][q] = *reinterpret_cast<const u32x4*>(base + fa_off[ks] + 4096 * q);
    else fw[set][q - MT] = *reinterpret_cast<const u32x4*>(base + fw_off[ks] + w_row[q - MT]);
  };

  const int last = (ke - 1) * BK;
#pragma unroll
  for (int i = 0; i < NCH; ++i) rg[i] = *gsrc(i, kb * BK);
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(smem + dst(i)) = rg[i];
#pragma unroll
  for (int i = 0; i < NCH; ++i) rg[i] = *gsrc(i, min((kb + 1) * BK, last));
  __syncthreads();
#pragma unroll
  for (int q = 0; q < MT + NT; ++q) rd1(smem, 0, 0, q);

  // Each k16 step issues, in this order and pinned by sched_barrier: MFMA q, fragment read q of
  // the next step (q < MT + NT), and for steps 0..2 one staging pair (LDS write of tile t+1,
  // global load of tile t+2). Step 3 follows the barrier and reads the next tile's step-0
  // fragments from the other buffer.
  for (int kt = kb; kt < ke; ++kt) {
    const int buf = (kt - kb) & 1;
    const uint8_t* ab = smem + buf * C::STAGE;
    uint8_t* nb = smem + (buf ^ 1) * C::STAGE;
    const int knext = min((kt + 2) * BK, last);  // past the end: re-read the last tile (unused)
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1, nx = cur ^ 1;
      if (ks == BK / 16 - 1) {
        // tile t+1 complete in the other buffer; every read of this buffer has been issued
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* rbase = (ks == BK / 16 - 1) ? nb : ab;
      const int rks = (ks == BK / 16 - 1) ? 0 : ks + 1;
#pragma unroll
      for (int q = 0; q < MT * NT; ++q) {
        acc[q / NT][q % NT] = mfma32x32x16(fa[cur][q / NT], fw[cur][q % NT], acc[q / NT][q % NT]);
        if (q < MT + NT) rd1(rbase, nx, rks, q);
        if (ks < BK / 16 - 1 && q < PER && ks * PER + q < NCH) {
          const int i = ks * PER + q;
          *reinterpret_cast<u32x4*>(nb + dst(i)) = rg[i];
          rg[i] = *gsrc(i, knext);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the next call (stream-K) or the epilogue reuses the LDS
  __syncthreads();
}

// Rows of the 32 x 32 block a lane holds: 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32.
HL_DEV int block_row(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// RoPE + KV append for 8 pairs of one staged row: `srow` points at the fp32 row of one head.
// Only decode tokens (`decode`) get the low half of q: decode attention alone reads it.
template <int HD>
HL_DEV void rope_store_row(const GemmEpi& ep, int gm, int gh, int blk, int slot, bool decode,
                           const float* srow, int c) {
  constexpr int half = HD / 2;
  const int Hq = ep.n_q_heads, Hkv = ep.n_kv_heads;
  float a[8], b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = srow[8 * c + e];
    b[e] = srow[half + 8 * c + e];
  }
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
    *reinterpret_cast<u32x4*>(ep.q_rot + o) = pack8(a);
    *reinterpret_cast<u32x4*>(ep.q_rot + o + half) = pack8(b);
    if (ep.q_lo && decode) {  // what bf16 dropped, so decode attention can use q to ~16 bits
      float la[8], lb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        la[e] = a[e] - bf2f(f2bf(a[e]));
        lb[e] = b[e] - bf2f(f2bf(b[e]));
      }
      *reinterpret_cast<u32x4*>(ep.q_lo + o) = pack8(la);
      *reinterpret_cast<u32x4*>(ep.q_lo + o + half) = pack8(lb);
    }
    return;
  }
  if (blk < 0) return;
  if (gh < Hq + Hkv) {
    hl_bf16* dst = ep.kpool + (((size_t)blk * Hkv + (gh - Hq)) * HL_BLOCK_SIZE + slot) * HD + 8 * c;
    *reinterpret_cast<u32x4*>(dst) = pack8(a);
    *reinterpret_cast<u32x4*>(dst + half) = pack8(b);
  } else {
    hl_bf16* dst = ep.vpool + ((size_t)blk * Hkv + (gh - Hq - Hkv)) * HD * HL_BLOCK_SIZE + slot;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dst[(size_t)(8 * c + e) * HL_BLOCK_SIZE] = (hl_bf16)f2bf(a[e]);
      dst[(size_t)(half + 8 * c + e) * HL_BLOCK_SIZE] = (hl_bf16)f2bf(b[e]);
    }
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
  const int lc = lane & 31;
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
  int seg = 0;
  do {
    const int tile = it / sc.nk;
    const int kb = SK ? it % sc.nk : 0;
    const int ke = SK ? min(sc.nk, kb + (it_end - it)) : sc.nk;
    const int mt = tile % sc.mtiles, nt = tile / sc.mtiles;
    const int m0 = mt * BM;
    f32x16 acc[MT][NT];
    mainloop<EPI, BM, BN>(A, W, M, N, K, mt, nt, kb, ke, smem, acc);
    it += ke - kb;
    if (SK && (kb != 0 || ke != sc.nk)) {
      // a piece of a split tile: raw fp32 partial for the fix-up kernel (slot 0 = the first
      // segment of this workgroup's run, slot 1 = its last)
      float* pdst = sc.part + ((size_t)run * 2 + (seg == 0 ? 0 : 1)) * BM * BN;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            pdst[(wm * CF::WM + i * 32 + block_row(lane, r)) * BN + wn * CF::WN + t * 32 + lc] = acc[i][t][r];
      ++seg;
      continue;
    }
    ++seg;
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
        for (int r = 0; r < 16; ++r) {
          const int row = wm * CF::WM + i * 32 + block_row(lane, r), gm = m0 + row;
          if (gm >= M) continue;
          const float rs = rs_sh[row];
#pragma unroll
          for (int t = 0; t < NT / 2; ++t) {
            const float g = acc[i][t][r] * rs, u = acc[i][t + NT / 2][r] * rs;
            C[(size_t)gm * half_n + nt * (BN / 2) + wn * (CF::WN / 2) + t * 32 + lc] =
                (hl_bf16)f2bf(silu(g) * u);
          }
        }
    } else if constexpr (EPI == kEpiRopeAppend) {
      // stage the scaled fp32 tile in LDS, then rotate / route whole 8-element runs; a 256-row
      // tile is staged one wave row (128 rows) at a time so the stage fits in the main-loop LDS
      constexpr int NPASS = BM > 128 ? 2 : 1, PROWS = BM / NPASS;
      float* st = reinterpret_cast<float*>(smem);
      constexpr int heads = BN / HD, chunks = HD / 16;
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        if (NPASS == 1 || wm == pass) {
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = wm * CF::WM + i * 32 + block_row(lane, r);
#pragma unroll
              for (int t = 0; t < NT; ++t)
                st[(row - pass * PROWS) * BN + wn * CF::WN + t * 32 + lc] = acc[i][t][r] * rs_sh[row];
            }
        }
        __syncthreads();
        for (int e = tid; e < PROWS * heads * chunks; e += kThreads) {
          const int c = e % chunks, rest = e / chunks, hi = rest % heads, rr = rest / heads;
          const int r = pass * PROWS + rr, gm = m0 + r;
          if (gm >= M) continue;
          rope_store_row<HD>(ep, gm, nt * heads + hi, blk_sh[r], pos_sh[r] & (HL_BLOCK_SIZE - 1),
                             (pos_sh[r] & hl::kDecodeBit) != 0, st + rr * BN + hi * HD, c);
        }
        if (NPASS > 1) __syncthreads();
      }
    } else {
      const hl_bf16* R = ep.residual;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * CF::WM + i * 32 + block_row(lane, r), gm = m0 + row;
          if (gm >= M) continue;
          const float rs = rs_sh[row];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const size_t o = (size_t)gm * N + nt * BN + wn * CF::WN + t * 32 + lc;
            float v = acc[i][t][r] * rs;
            if (EPI == HL_EPI_RESIDUAL) v += bf2f(R[o]);
            C[o] = (hl_bf16)f2bf(v);
          }
        }
    }
    if constexpr (SK) __syncthreads();  // rs_sh / LDS reuse by the next segment
  } while (SK && it < it_end);
}

// Stream-K fix-up: for each split tile, sum its pieces and apply the plain or residual epilogue
// (stream-K is used only for those). Block (tile, y) covers 1024 / BN rows of the tile; each thread
// takes 4 consecutive columns (16-byte piece loads), so the grid has enough independent loads in
// flight.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(hl_bf16* __restrict__ C, int M, int N,
                                                         GemmEpi ep, Sched sc) {
  constexpr int TPR = BN / 4, RPB = 256 / TPR;  // threads per row, rows per block
  const int tile = blockIdx.x;
  const int first = tile * sc.nk, lastit = first + sc.nk - 1;
  const int w0 = first / sc.ipw, w1 = lastit / sc.ipw;
  if (w0 == w1) return;  // finished in one piece by the main kernel
  const int mt = tile % sc.mtiles, nt = tile / sc.mtiles;
  const int row = blockIdx.y * RPB + threadIdx.x / TPR, col = (threadIdx.x % TPR) * 4;
  const int gm = mt * BM + row;
  if (gm >= M) return;
  const int e = row * BN + col;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int w = w0; w <= w1; ++w) {
    const int slot = ((w * sc.ipw) / sc.nk == tile) ? 0 : 1;  // first segment of w's run?
    v += *reinterpret_cast<const f32x4*>(sc.part + ((size_t)w * 2 + slot) * BM * BN + e);
  }
  const size_t o = (size_t)gm * N + nt * BN + col;
  if (ep.row_scale) v *= ep.row_scale[gm];
  if (ep.kind == HL_EPI_RESIDUAL) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(ep.residual + o);
    v[0] += bf_lo(r[0]);
    v[1] += bf_hi(r[0]);
    v[2] += bf_lo(r[1]);
    v[3] += bf_hi(r[1]);
  }
  *reinterpret_cast<u32x2*>(C + o) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
}

template <int EPI, int BM, int BN, int HD = 0>
hipError_t launch_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, float* part, bool streamk, hipStream_t st) {
  using CF = Cfg<BM, BN>;
  constexpr bool kCanSplit = (EPI == HL_EPI_NONE || EPI == HL_EPI_RESIDUAL);
  auto kern = gemm_bf16_nt_kernel<EPI, BM, BN, HD, false>;
  auto kern_sk = gemm_bf16_nt_kernel<EPI, BM, BN, HD, kCanSplit>;
  const int lds = (EPI == kEpiRopeAppend) ? max(CF::MAIN_LDS, min(BM, 128) * BN * 4) : CF::MAIN_LDS;
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
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, st, a, w, c, m, n, k, epi, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !streamk) return e;
  hipLaunchKernelGGL((gemm_fixup_kernel<BM, BN>), dim3(tiles, BM / (1024 / BN)), dim3(256), 0, st,
                     c, m, n, epi, sc);
  return hipGetLastError();
}

// Schedule of a plain / residual GEMM. Measured on the layer shapes: stream-K over 128 x 256 tiles
// is the best or close to it everywhere (it fills every CU, and its pieces are small), except for
// the long-K down projections, where 256 x 256 tiles (1.5x less LDS and L2 traffic per flop) win
// once each workgroup's run is long enough to hide the larger pieces. Without a workspace, or when
// the 128 x 256 tiles fill whole rounds: one tile per workgroup.
struct PlainChoice {
  bool wide;     // 256 x 256 tiles (else 128 x 256)
  bool streamk;
};
PlainChoice choose_plain(int m, int n, int k, bool has_ws) {
  const int nk = k / BK;
  if (!has_ws || nk < 4) return PlainChoice{false, false};
  const long narrow_tiles = (long)((m + 127) / 128) * (n / 256);
  const long wide_tiles = (long)((m + 255) / 256) * (n / 256);
  const long narrow_run = (narrow_tiles * nk + kStreamKGrid - 1) / kStreamKGrid;
  const long wide_run = (wide_tiles * nk + kStreamKGrid - 1) / kStreamKGrid;
  if (m > 128 && narrow_run >= 384 && wide_run >= 200) return PlainChoice{true, true};
  return PlainChoice{false, narrow_tiles % kStreamKGrid != 0};
}

// One tile per workgroup (SwiGLU and RoPE epilogues): 256 x 256 tiles when their rounds, at 1.5x
// the time of a 128 x 256 round (the measured ratio of k-step times), finish first.
bool wide_one_tile(int m, int n) {
  if (n % 256 != 0 || m <= 128) return false;
  const long rn = ((long)((m + 127) / 128) * (n / 256) + kStreamKGrid - 1) / kStreamKGrid;
  const long rw = ((long)((m + 255) / 256) * (n / 256) + kStreamKGrid - 1) / kStreamKGrid;
  return 3 * rw < 2 * rn;
}

template <int EPI>
hipError_t launch_plain(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, float* part, size_t ws_bytes, hipStream_t st) {
  if (n % 256 != 0) return launch_tiles<EPI, 128, 128>(a, w, c, m, n, k, epi, nullptr, false, st);
  const PlainChoice ch = choose_plain(m, n, k, part && ws_bytes >= kStreamKWorkspace);
  if (ch.wide) return launch_tiles<EPI, 256, 256>(a, w, c, m, n, k, epi, part, ch.streamk, st);
  return launch_tiles<EPI, 128, 256>(a, w, c, m, n, k, epi, part, ch.streamk, st);
}

}  // namespace

namespace hl {

// Stream-K pieces: up to kStreamKGrid workgroups x 2 pieces x a 256 x 256 fp32 tile.
size_t gemm_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return kStreamKWorkspace; }

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  float* part = static_cast<float*>(ws);
  switch (epi.kind) {
    case HL_EPI_NONE:
      return launch_plain<HL_EPI_NONE>(a, w, c, m, n, k, epi, part, ws_bytes, st);
    case HL_EPI_RESIDUAL:
      return launch_plain<HL_EPI_RESIDUAL>(a, w, c, m, n, k, epi, part, ws_bytes, st);
    case HL_EPI_SWIGLU:
      if (wide_one_tile(m, n)) return launch_tiles<HL_EPI_SWIGLU, 256, 256>(a, w, c, m, n, k, epi, nullptr, false, st);
      if (n % 256 == 0) return launch_tiles<HL_EPI_SWIGLU, 128, 256>(a, w, c, m, n, k, epi, nullptr, false, st);
      return launch_tiles<HL_EPI_SWIGLU, 128, 128>(a, w, c, m, n, k, epi, nullptr, false, st);
    default:
      if (wide_one_tile(m, n))
        return epi.head_dim == 128
                   ? launch_tiles<kEpiRopeAppend, 256, 256, 128>(a, w, c, m, n, k, epi, nullptr, false, st)
                   : launch_tiles<kEpiRopeAppend, 256, 256, 64>(a, w, c, m, n, k, epi, nullptr, false, st);
      return epi.head_dim == 128
                 ? launch_tiles<kEpiRopeAppend, 128, 256, 128>(a, w, c, m, n, k, epi, nullptr, false, st)
                 : launch_tiles<kEpiRopeAppend, 128, 256, 64>(a, w, c, m, n, k, epi, nullptr, false, st);
  }
}

}  // namespace hl
