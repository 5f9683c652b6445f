// Token-batched linear layer on the CDNA4 matrix cores: C = A W^T (bf16 in, fp32 accumulate).
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?").
//
// Main loop (512 threads = 8 waves, 2 per SIMD; K advances 64 per tile). A and W tiles are staged
// through LDS in 128-byte rows whose 16-byte chunks are XOR-swizzled with (row / 2) mod 8, which
// keeps every 16-lane group of a fragment read on distinct banks. Each wave owns a grid of
// v_mfma_f32_32x32x16_bf16 blocks. One register staging set: while the matrix cores work on tile
// t, the wave reads the fragments of the next k16 step (double-buffered fragments) and, during the
// last step, writes tile t+1 into the other LDS buffer and issues the global loads of tile t+2;
// sched_group_barrier threads these memory instructions between the MFMAs instead of leaving them
// in phases of their own (measured on gfx950: ~1.3x over a phased loop). Tiles are dealt so that
// consecutive tile ids land on the same XCD (workgroups go to the 8 XCDs round-robin) and, within
// an XCD, the M tiles of one N column run together, so a weight tile is fetched from HBM once.
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

constexpr int BK = 64, kThreads = 512, kWaves = 8;

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
  float* part;             // stream-K: [grid][2][BM * BN] fp32 pieces
};

template <int BM, int BN, int WAVES_M>
struct Cfg {
  static constexpr int WAVES_N = kWaves / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MT = WM / 32, NT = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int A_CH = A_BYTES / 16 / kThreads, W_CH = W_BYTES / 16 / kThreads;
  static constexpr int NCH = A_CH + W_CH;
  static constexpr int MAIN_LDS = 2 * STAGE;
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
template <int EPI, int BM, int BN, int WAVES_M>
HL_DEV void mainloop(const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, int M, int N,
                     int K, int mt, int nt, int kb, int ke, uint8_t* smem,
                     f32x16 (&acc)[Cfg<BM, BN, WAVES_M>::MT][Cfg<BM, BN, WAVES_M>::NT]) {
  using C = Cfg<BM, BN, WAVES_M>;
  constexpr int MT = C::MT, NT = C::NT, NCH = C::NCH, A_CH = C::A_CH, NMF = MT * NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int m0 = mt * BM;
  const int half_n = N >> 1;

  // Global sources. Rows past M read row M-1: a C row depends only on its own A row and padded
  // C rows are never stored, so the loads need no branch.
  const hl_bf16* src[NCH];
  int dst_off[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (i < A_CH) {
      const int q = tid + kThreads * i, row = q >> 3, ch = q & 7;
      src[i] = A + (size_t)min(m0 + row, M - 1) * K + ch * 8;
      dst_off[i] = swz(row, ch);
    } else {
      const int q = tid + kThreads * (i - A_CH), row = q >> 3, ch = q & 7;
      int wr;
      if (EPI == HL_EPI_SWIGLU)
        wr = (row < BN / 2) ? nt * (BN / 2) + row : half_n + nt * (BN / 2) + (row - BN / 2);
      else
        wr = nt * BN + row;
      src[i] = W + (size_t)wr * K + ch * 8;
      dst_off[i] = C::A_BYTES + swz(row, ch);
    }
  }
  int a_off[MT], w_off[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i) a_off[i] = wm * C::WM + i * 32 + (lane & 31);
#pragma unroll
  for (int t = 0; t < NT; ++t) w_off[t] = w_block_row<EPI, BN, C::WN, NT>(wn, t) + (lane & 31);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x16{};

  const int last = (ke - 1) * BK;
  u32x4 rg[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) rg[i] = *reinterpret_cast<const u32x4*>(src[i] + kb * BK);
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(smem + dst_off[i]) = rg[i];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    rg[i] = *reinterpret_cast<const u32x4*>(src[i] + min((kb + 1) * BK, last));
  __syncthreads();

  for (int kt = kb; kt < ke; ++kt) {
    const int buf = (kt - kb) & 1;
    const uint8_t* ab = smem + buf * C::STAGE;
    const uint8_t* wb = ab + C::A_BYTES;
    uint8_t* nb = smem + (buf ^ 1) * C::STAGE;
    const int knext = min((kt + 2) * BK, last);  // past the end: re-read the last tile (unused)
    u32x4 fa[2][MT], fw[2][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) fa[0][i] = *reinterpret_cast<const u32x4*>(ab + swz(a_off[i], lane >> 5));
#pragma unroll
    for (int t = 0; t < NT; ++t) fw[0][t] = *reinterpret_cast<const u32x4*>(wb + swz(w_off[t], lane >> 5));
    __builtin_amdgcn_sched_group_barrier(0x100, MT + NT, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma32x32x16(fa[cur][i], fw[cur][t], acc[i][t]);
      if (ks + 1 < BK / 16) {
        const int ch = 2 * (ks + 1) + (lane >> 5);
#pragma unroll
        for (int i = 0; i < MT; ++i) fa[cur ^ 1][i] = *reinterpret_cast<const u32x4*>(ab + swz(a_off[i], ch));
#pragma unroll
        for (int t = 0; t < NT; ++t) fw[cur ^ 1][t] = *reinterpret_cast<const u32x4*>(wb + swz(w_off[t], ch));
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
          if (q < MT + NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(nb + dst_off[i]) = rg[i];
#pragma unroll
        for (int i = 0; i < NCH; ++i) rg[i] = *reinterpret_cast<const u32x4*>(src[i] + knext);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
          if (q < NCH) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);          // LDS write
          else if (q < 2 * NCH) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        }
      }
    }
    __syncthreads();
  }
}

// Rows of the 32 x 32 block a lane holds: 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32.
HL_DEV int block_row(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// RoPE + KV append for 8 pairs of one staged row: `srow` points at the fp32 row of one head.
template <int HD>
HL_DEV void rope_store_row(const GemmEpi& ep, int gm, int gh, int blk, int slot, const float* srow,
                           int c) {
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
    if (ep.q_lo) {  // what bf16 dropped, so decode attention can use q to ~16 bits
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
template <int EPI, int BM, int BN, int WAVES_M, int HD, bool SK>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_nt_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, hl_bf16* __restrict__ C, int M,
    int N, int K, GemmEpi ep, Sched sc) {
  using CF = Cfg<BM, BN, WAVES_M>;
  constexpr int MT = CF::MT, NT = CF::NT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float rs_sh[BM];
  __shared__ int pos_sh[BM];
  __shared__ int blk_sh[BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  const int lc = lane & 31;
  const int half_n = N >> 1;
  const int tiles = sc.mtiles * sc.ntiles;

  // work: one tile, or a stream-K run of (tile, k-step) iterations
  int it = 0, it_end = 0;
  if constexpr (!SK) {
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    it = tile * sc.nk;
    it_end = it + sc.nk;
  } else {
    it = blockIdx.x * sc.ipw;
    it_end = min(it + sc.ipw, tiles * sc.nk);
  }
  int seg = 0;
  while (it < it_end) {
    const int tile = it / sc.nk;
    const int kb = SK ? it % sc.nk : 0;
    const int ke = SK ? min(sc.nk, kb + (it_end - it)) : sc.nk;
    const int mt = tile % sc.mtiles, nt = tile / sc.mtiles;
    const int m0 = mt * BM;
    f32x16 acc[MT][NT];
    mainloop<EPI, BM, BN, WAVES_M>(A, W, M, N, K, mt, nt, kb, ke, smem, acc);
    it += ke - kb;
    if (SK && (kb != 0 || ke != sc.nk)) {
      // a piece of a split tile: raw fp32 partial for the fix-up kernel (slot 0 = the first
      // segment of this workgroup's run, slot 1 = its last)
      float* pdst = sc.part + ((size_t)blockIdx.x * 2 + (seg == 0 ? 0 : 1)) * BM * BN;
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
      // stage the scaled fp32 tile in LDS, then rotate / route whole 8-element runs
      float* st = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * CF::WM + i * 32 + block_row(lane, r);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            st[row * BN + wn * CF::WN + t * 32 + lc] = acc[i][t][r] * rs_sh[row];
        }
      __syncthreads();
      constexpr int heads = BN / HD, chunks = HD / 16;
      for (int e = tid; e < BM * heads * chunks; e += kThreads) {
        const int c = e % chunks, rest = e / chunks, hi = rest % heads, r = rest / heads;
        const int gm = m0 + r;
        if (gm >= M) continue;
        rope_store_row<HD>(ep, gm, nt * heads + hi, blk_sh[r], pos_sh[r] & (HL_BLOCK_SIZE - 1),
                           st + r * BN + hi * HD, c);
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
    if constexpr (!SK) break;
    __syncthreads();  // rs_sh / LDS reuse by the next segment
  }
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

template <int EPI, int BM, int BN, int WAVES_M, int HD = 0>
hipError_t launch_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, float* part, size_t part_bytes, hipStream_t st) {
  using CF = Cfg<BM, BN, WAVES_M>;
  constexpr bool kCanSplit = (EPI == HL_EPI_NONE || EPI == HL_EPI_RESIDUAL);
  auto kern = gemm_bf16_nt_kernel<EPI, BM, BN, WAVES_M, HD, false>;
  auto kern_sk = gemm_bf16_nt_kernel<EPI, BM, BN, WAVES_M, HD, kCanSplit>;
  const int lds = (EPI == kEpiRopeAppend) ? max(CF::MAIN_LDS, BM * BN * 4) : CF::MAIN_LDS;
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
  sc.part = part;
  const int tiles = sc.mtiles * sc.ntiles;
  int grid = tiles;
  // stream-K when the tiles leave compute units idle and the workspace can hold the pieces
  const int cus = 256;
  const bool streamk = kCanSplit && tiles < cus &&
                       part && part_bytes >= (size_t)cus * 2 * BM * BN * 4 && sc.nk >= 4;
  if (streamk) {
    const int total = tiles * sc.nk;
    sc.ipw = (total + cus - 1) / cus;
    grid = (total + sc.ipw - 1) / sc.ipw;
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

}  // namespace

namespace hl {

// Stream-K pieces of the narrow GEMMs: 256 workgroups x 2 pieces x a 128 x 256 fp32 tile.
size_t gemm_workspace_bytes(int32_t, int32_t, int32_t, int32_t) {
  return (size_t)256 * 2 * 128 * 256 * 4;
}

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  float* part = static_cast<float*>(ws);
  switch (epi.kind) {
    case HL_EPI_NONE:
      if (n % 256 == 0) return launch_tiles<HL_EPI_NONE, 128, 256, 2>(a, w, c, m, n, k, epi, part, ws_bytes, st);
      return launch_tiles<HL_EPI_NONE, 128, 128, 4>(a, w, c, m, n, k, epi, part, ws_bytes, st);
    case HL_EPI_RESIDUAL:
      if (n % 256 == 0) return launch_tiles<HL_EPI_RESIDUAL, 128, 256, 2>(a, w, c, m, n, k, epi, part, ws_bytes, st);
      return launch_tiles<HL_EPI_RESIDUAL, 128, 128, 4>(a, w, c, m, n, k, epi, part, ws_bytes, st);
    case HL_EPI_SWIGLU:
      if (n % 256 == 0 && m > 512) return launch_tiles<HL_EPI_SWIGLU, 256, 256, 4>(a, w, c, m, n, k, epi, nullptr, 0, st);
      if (n % 256 == 0) return launch_tiles<HL_EPI_SWIGLU, 128, 256, 2>(a, w, c, m, n, k, epi, nullptr, 0, st);
      return launch_tiles<HL_EPI_SWIGLU, 128, 128, 4>(a, w, c, m, n, k, epi, nullptr, 0, st);
    default:
      return epi.head_dim == 128
                 ? launch_tiles<kEpiRopeAppend, 128, 256, 2, 128>(a, w, c, m, n, k, epi, nullptr, 0, st)
                 : launch_tiles<kEpiRopeAppend, 128, 256, 2, 64>(a, w, c, m, n, k, epi, nullptr, 0, st);
  }
}

}  // namespace hl
