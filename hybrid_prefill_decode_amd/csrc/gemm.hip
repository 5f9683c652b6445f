// Token-batched linear layer on the CDNA4 matrix cores: C = A W^T (bf16 in, fp32 accumulate).
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?").
//
// Tiling. A 256-thread workgroup computes a 128 x BN tile of C (BN = 256 for wide N, 128 for
// narrow N); K advances 32 at a time. The 4 waves form a 2 x 2 grid, each owning 64 x BN/2 =
// 2 x BN/64 blocks of v_mfma_f32_32x32x16_bf16, so every 16-byte fragment read from LDS feeds
// more than one matrix-core op (the LDS, not the matrix cores, limits a 64 x 64 wave tile on
// gfx950). A and W tiles are staged through LDS in 64-byte rows whose 16-byte chunks are
// XOR-swizzled with (row / 4) mod 4, which keeps every group of 16 lanes reading one fragment on
// distinct banks. Global loads run two tiles ahead through two register staging sets (the loop is
// unrolled by two so the sets are named statically, and every load is issued unconditionally so
// the wait counts follow the pipeline). Tiles are dealt so that consecutive tile ids land on the
// same XCD (workgroups go to the 8 XCDs round-robin) and, within an XCD, the M tiles of one N
// column run together, so a weight tile is fetched from HBM about once.
//
// Epilogues work on the accumulators in registers, after an optional per-row scale (the RMSNorm
// factor, see prep.hip): plain, + residual, SwiGLU (the W tile holds BN/2 gate rows and the
// matching BN/2 up rows; each lane holds a gate and its up in registers), and RoPE + KV append for
// the QKV projection (each lane holds the pair (j, j + d/2) of a head in registers: q heads are
// rotated into q_rot, k heads rotated and v heads copied into their cache pages).
#include "common.h"

namespace {
using hl::GemmEpi;
using hl::kEpiRopeAppend;

constexpr int BM = 128, BK = 32, kThreads = 256;

// 64-byte LDS rows (32 bf16 of K); 16-byte chunk c of row r lives at chunk c ^ ((r >> 2) & 3)
HL_DEV int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

// Bijection from dispatch order to tile order that keeps consecutive tiles on one XCD.
HL_DEV int xcd_tile(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// HD: head dim, compile-time for the RoPE epilogue (so the pair of a lane is a static register
// pair); unused by the other epilogues.
template <int EPI, int BN, int HD>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_nt_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, hl_bf16* __restrict__ C, int M,
    int N, int K, int mtiles, GemmEpi ep) {
  constexpr int WN = BN / 2;             // wave tile N
  constexpr int NT = WN / 32;            // 32-wide blocks per wave in N
  constexpr int A_BYTES = BM * BK * 2;   // 8 KB
  constexpr int W_BYTES = BN * BK * 2;   // 8 or 16 KB
  constexpr int STAGE = A_BYTES + W_BYTES;
  constexpr int A_CH = A_BYTES / 16 / kThreads;  // 16-byte chunks per thread
  constexpr int W_CH = W_BYTES / 16 / kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ float rs_sh[BM];
  __shared__ int pos_sh[BM];
  __shared__ int blk_sh[BM];

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half_n = N >> 1;  // SwiGLU: gate rows [0, half_n), up rows [half_n, N)

  if (tid < BM) {
    const int gm = m0 + tid;
    rs_sh[tid] = (ep.row_scale && gm < M) ? ep.row_scale[gm] : 1.f;
    if (EPI == kEpiRopeAppend) {
      pos_sh[tid] = gm < M ? ep.tok_pos[gm] : 0;
      blk_sh[tid] = gm < M ? ep.tok_blk[gm] : -1;
    }
  }

  // Global sources. Rows past M read row M-1: a C row depends only on its own A row and padded
  // C rows are never stored, so the loads need no branch.
  const hl_bf16* a_src[A_CH];
  const hl_bf16* w_src[W_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = tid + kThreads * i, row = q >> 2, ch = q & 3;
    a_src[i] = A + (size_t)min(m0 + row, M - 1) * K + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < W_CH; ++i) {
    const int q = tid + kThreads * i, row = q >> 2, ch = q & 3;
    int wr;
    if (EPI == HL_EPI_SWIGLU)
      wr = (row < BN / 2) ? nt * (BN / 2) + row : half_n + nt * (BN / 2) + (row - BN / 2);
    else
      wr = nt * BN + row;
    w_src[i] = W + (size_t)wr * K + ch * 8;
  }

  u32x4 ra[2][A_CH], rw[2][W_CH];
  auto gload = [&](int set, int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[set][i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < W_CH; ++i) rw[set][i] = *reinterpret_cast<const u32x4*>(w_src[i] + k0);
  };
  auto sstore = [&](int buf, int set) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(base + swz(q >> 2, q & 3)) = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(base + A_BYTES + swz(q >> 2, q & 3)) = rw[set][i];
    }
  };

  // W-tile row of this wave's block t (SwiGLU pairs gate block t with up block t + NT/2)
  auto w_block_row = [&](int t) {
    if (EPI == HL_EPI_SWIGLU)
      return (t < NT / 2) ? wn * (BN / 4) + t * 32 : BN / 2 + wn * (BN / 4) + (t - NT / 2) * 32;
    return wn * WN + t * 32;
  };
  int a_row[2], w_row[NT];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_row[i] = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
  for (int t = 0; t < NT; ++t) w_row[t] = w_block_row(t) + (lane & 31);

  f32x16 acc[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x16{};

  auto compute = [&](int buf) {
    const uint8_t* a_base = smem + buf * STAGE;
    const uint8_t* w_base = a_base + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      u32x4 fa[2], fw[NT];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const u32x4*>(a_base + swz(a_row[i], ch));
#pragma unroll
      for (int t = 0; t < NT; ++t) fw[t] = *reinterpret_cast<const u32x4*>(w_base + swz(w_row[t], ch));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma32x32x16(fa[i], fw[t], acc[i][t]);
    }
  };

  // K % 64 == 0, so the tile count is even and the two-way unrolled loop needs no early exit.
  // Tile t lives in register set t & 1 and LDS buffer t & 1, and goes to LDS while tile t-1 is
  // multiplied. Past the end the prefetches re-read the last tile (valid addresses, unused).
  // sched_barrier keeps the scheduler from merging the phases, which would make the LDS stores
  // wait for the younger loads as well.
  const int nk = K / BK;
  const int last = (nk - 1) * BK;
  gload(0, 0);
  gload(1, BK);
  sstore(0, 0);
  __syncthreads();
  gload(0, min(2 * BK, last));
  for (int kt = 0; kt < nk; kt += 2) {
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    sstore(1, 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    gload(1, min((kt + 3) * BK, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    sstore(0, 0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    gload(0, min((kt + 4) * BK, last));
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue from registers: lane holds rows 8 (r / 4) + 4 (lane / 32) + r % 4 of each
  // 32 x 32 block, column lane % 32
  const int lc = lane & 31;
  auto row_of = [&](int i, int r) { return wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };

  if (EPI == HL_EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_of(i, r), gm = m0 + row;
        if (gm >= M) continue;
        const float rs = rs_sh[row];
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
          const float g = acc[i][t][r] * rs, u = acc[i][t + NT / 2][r] * rs;
          const float sv = g / (1.f + __expf(-g));
          C[(size_t)gm * half_n + nt * (BN / 2) + wn * (BN / 4) + t * 32 + lc] = (hl_bf16)f2bf(sv * u);
        }
      }
  } else if (EPI == kEpiRopeAppend) {
    constexpr int D = HD, half = D / 2;
    const int Hq = ep.n_q_heads, Hkv = ep.n_kv_heads;
    constexpr int bph = D / 32;   // 32-wide blocks per head
    const int col0 = nt * BN + wn * WN;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tt = t % bph;
      if (tt >= bph / 2) continue;  // second halves are handled with their first halves
      const int tp = t + bph / 2;
      const int gh = (col0 + t * 32) / D;
      const int j = tt * 32 + lc;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_of(i, r), gm = m0 + row;
          if (gm >= M) continue;
          const float rs = rs_sh[row];
          float a = acc[i][t][r] * rs, b = acc[i][tp][r] * rs;
          if (gh < Hq + Hkv) {
            const float2 cs = ep.rope_cs[(size_t)gm * half + j];
            const float ra = a * cs.x - b * cs.y, rb = b * cs.x + a * cs.y;
            a = ra;
            b = rb;
          }
          if (gh < Hq) {
            const size_t o = ((size_t)gm * Hq + gh) * D + j;
            const uint32_t ha = f2bf(a), hb = f2bf(b);
            ep.q_rot[o] = (hl_bf16)ha;
            ep.q_rot[o + half] = (hl_bf16)hb;
            if (ep.q_lo) {  // what bf16 dropped, so decode attention can use q to ~16 bits
              ep.q_lo[o] = (hl_bf16)f2bf(a - bf2f(ha));
              ep.q_lo[o + half] = (hl_bf16)f2bf(b - bf2f(hb));
            }
            continue;
          }
          const int blk = blk_sh[row];
          if (blk < 0) continue;
          const int slot = pos_sh[row] & (HL_BLOCK_SIZE - 1);
          if (gh < Hq + Hkv) {
            hl_bf16* dst = ep.kpool + (((size_t)blk * Hkv + (gh - Hq)) * HL_BLOCK_SIZE + slot) * D;
            dst[j] = (hl_bf16)f2bf(a);
            dst[j + half] = (hl_bf16)f2bf(b);
          } else {
            hl_bf16* dst = ep.vpool + ((size_t)blk * Hkv + (gh - Hq - Hkv)) * D * HL_BLOCK_SIZE + slot;
            dst[(size_t)j * HL_BLOCK_SIZE] = (hl_bf16)f2bf(a);
            dst[(size_t)(j + half) * HL_BLOCK_SIZE] = (hl_bf16)f2bf(b);
          }
        }
    }
  } else {
    const hl_bf16* R = ep.residual;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_of(i, r), gm = m0 + row;
        if (gm >= M) continue;
        const float rs = rs_sh[row];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const size_t o = (size_t)gm * N + nt * BN + wn * WN + t * 32 + lc;
          float v = acc[i][t][r] * rs;
          if (EPI == HL_EPI_RESIDUAL) v += bf2f(R[o]);
          C[o] = (hl_bf16)f2bf(v);
        }
      }
  }
}

template <int EPI, int BN, int HD = 0>
hipError_t launch_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int m, int n, int k,
                        const GemmEpi& epi, hipStream_t st) {
  const int mtiles = (m + BM - 1) / BM;
  const int ntiles = n / BN;
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<EPI, BN, HD>), dim3(mtiles * ntiles), dim3(kThreads), 0,
                     st, a, w, c, m, n, k, mtiles, epi);
  return hipGetLastError();
}

}  // namespace

namespace hl {

size_t gemm_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void*, size_t, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  // 256-wide tiles when N leaves enough of them to fill the chip; RoPE needs a whole head per wave
  const int mtiles = (m + BM - 1) / BM;
  const bool wide = (n % 256 == 0) &&
                    (epi.kind == kEpiRopeAppend || (int64_t)mtiles * (n / 256) >= 512);
  switch (epi.kind) {
    case HL_EPI_NONE:
      return wide ? launch_tiles<HL_EPI_NONE, 256>(a, w, c, m, n, k, epi, st)
                  : launch_tiles<HL_EPI_NONE, 128>(a, w, c, m, n, k, epi, st);
    case HL_EPI_RESIDUAL:
      return wide ? launch_tiles<HL_EPI_RESIDUAL, 256>(a, w, c, m, n, k, epi, st)
                  : launch_tiles<HL_EPI_RESIDUAL, 128>(a, w, c, m, n, k, epi, st);
    case HL_EPI_SWIGLU:
      return wide ? launch_tiles<HL_EPI_SWIGLU, 256>(a, w, c, m, n, k, epi, st)
                  : launch_tiles<HL_EPI_SWIGLU, 128>(a, w, c, m, n, k, epi, st);
    default:
      return epi.head_dim == 128 ? launch_tiles<kEpiRopeAppend, 256, 128>(a, w, c, m, n, k, epi, st)
                                 : launch_tiles<kEpiRopeAppend, 256, 64>(a, w, c, m, n, k, epi, st);
  }
}

}  // namespace hl
