// Token-batched linear layer on the CDNA4 matrix cores: C = A W^T (bf16 in, fp32 accumulate).
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?").
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C with K stepped 64 at a time;
// A and W tiles are staged through LDS (XOR-swizzled 16-byte chunks, double buffered, next tile
// prefetched into registers while the matrix cores work on the current one); each of the 4
// waves owns a 64 x 64 sub-tile = 2 x 2 blocks of v_mfma_f32_32x32x16_bf16. Tiles are dealt so
// that consecutive tile ids land on the same XCD (workgroups are handed to the 8 XCDs
// round-robin), and within an XCD the M tiles of one N column run together, so each weight tile
// is fetched from HBM about once. Epilogues run on the fp32 tile staged in LDS, after an optional
// per-row scale (the RMSNorm factor, see prep.hip): plain, + residual, SwiGLU (the 128-row W tile
// holds 64 gate rows and the matching 64 up rows), and RoPE + KV append for the QKV projection
// (q heads rotated into q_rot, k heads rotated and v heads copied into their cache pages, so the
// unrotated q/k/v never go to memory).
#include "common.h"

namespace {
using hl::GemmEpi;
using hl::kEpiRopeAppend;

constexpr int BM = 128, BN = 128, BK = 64, kThreads = 256;
constexpr int kTileBytes = 128 * BK * 2;         // one 128 x 64 bf16 operand tile
constexpr int kStageBytes = 2 * kTileBytes;      // A + W
constexpr int kSmemBytes = 2 * kStageBytes;      // double buffered: 64 KB
constexpr int kRowInfoBytes = 3 * BM * 4;         // row scale, position, block of the tile rows
constexpr int kSmemTotal = kSmemBytes + kRowInfoBytes;

HL_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Bijection from dispatch order to tile order that keeps consecutive tiles on one XCD.
HL_DEV int xcd_tile(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

HL_DEV void store_bf16x8(hl_bf16* dst, const float* v) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
  *reinterpret_cast<u32x4*>(dst) = o;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_nt_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, hl_bf16* __restrict__ C, int M,
    int N, int K, int mtiles, GemmEpi ep) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* rs_sh = reinterpret_cast<float*>(smem + kSmemBytes);
  int* pos_sh = reinterpret_cast<int*>(smem + kSmemBytes + BM * 4);
  int* blk_sh = reinterpret_cast<int*>(smem + kSmemBytes + 2 * BM * 4);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < BM) {
    const int gm = m0 + tid;
    rs_sh[tid] = (ep.row_scale && gm < M) ? ep.row_scale[gm] : 1.f;
    if (EPI == kEpiRopeAppend) {
      pos_sh[tid] = gm < M ? ep.tok_pos[gm] : 0;
      blk_sh[tid] = gm < M ? ep.tok_blk[gm] : -1;
    }
  }
  const int wm = wave >> 1, wn = wave & 1;
  const int half_n = N >> 1;  // SwiGLU: gate rows [0, half_n), up rows [half_n, N)

  // global -> register staging: 4 x 16 B of A and 4 x 16 B of W per thread
  const hl_bf16* a_src[4];
  const hl_bf16* w_src[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + kThreads * i, row = q >> 3, ch = q & 7;
    const int gm = m0 + row;
    a_ok[i] = gm < M;
    a_src[i] = A + (size_t)(a_ok[i] ? gm : 0) * K + ch * 8;
    int wr;
    if (EPI == HL_EPI_SWIGLU)
      wr = (row < 64) ? nt * 64 + row : half_n + nt * 64 + (row - 64);
    else
      wr = nt * BN + row;
    w_src[i] = W + (size_t)wr * K + ch * 8;
  }
  u32x4 ra[4], rw[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : u32x4{0, 0, 0, 0};
      rw[i] = *reinterpret_cast<const u32x4*>(w_src[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + kThreads * i, row = q >> 3, ch = q & 7;
      *reinterpret_cast<u32x4*>(base + swz(row, ch)) = ra[i];
      *reinterpret_cast<u32x4*>(base + kTileBytes + swz(row, ch)) = rw[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // rows this wave reads from the staged tiles
  int a_row[2], w_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_row[i] = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    w_row[t] = (EPI == HL_EPI_SWIGLU ? t * 64 + wn * 32 : wn * 64 + t * 32) + (lane & 31);

  const int nk = K / BK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    sstore(buf);
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint8_t* a_base = smem + buf * kStageBytes;
    const uint8_t* w_base = a_base + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      u32x4 fa[2], fw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(a_base + swz(a_row[i], ch));
#pragma unroll
      for (int t = 0; t < 2; ++t)
        fw[t] = *reinterpret_cast<const u32x4*>(w_base + swz(w_row[t], ch));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[i][t] = mfma32x32x16(fa[i], fw[t], acc[i][t]);
    }
  }
  __syncthreads();  // all waves are done reading the operand tiles; reuse LDS for the epilogue

  // stage fp32 results: [128 rows][OUT_N cols]
  constexpr int OUT_N = (EPI == HL_EPI_SWIGLU) ? 64 : 128;
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const float rs = rs_sh[row];
      if (EPI == HL_EPI_SWIGLU) {
        const float g = acc[i][0][r] * rs, u = acc[i][1][r] * rs;
        const float s = g / (1.f + __expf(-g));
        st[row * OUT_N + wn * 32 + (lane & 31)] = s * u;
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          st[row * OUT_N + wn * 64 + t * 32 + (lane & 31)] = acc[i][t][r] * rs;
      }
    }
  }
  __syncthreads();
  if (EPI == kEpiRopeAppend) {
    // heads of this tile: q heads -> q_rot, k heads -> K pages (rotated), v heads -> V pages
    const int D = ep.head_dim, half = D >> 1, chunks = half >> 3;
    const int heads = BN / D, h0 = nt * heads;
    const int Hq = ep.n_q_heads, Hkv = ep.n_kv_heads;
    for (int it = tid; it < BM * heads * chunks; it += kThreads) {
      const int c = it % chunks, rest = it / chunks, hi = rest % heads, r = rest / heads;
      const int gm = m0 + r;
      if (gm >= M) continue;
      const int gh = h0 + hi;
      const float* srow = st + r * BN + hi * D;
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
      if (gh < Hq) {
        hl_bf16* dst = ep.q_rot + ((size_t)gm * Hq + gh) * D;
        store_bf16x8(dst + 8 * c, a);
        store_bf16x8(dst + half + 8 * c, b);
        if (ep.q_lo) {  // what bf16 dropped, so decode attention can use q to ~16 bits
          float la[8], lb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            la[e] = a[e] - bf2f(f2bf(a[e]));
            lb[e] = b[e] - bf2f(f2bf(b[e]));
          }
          hl_bf16* lo = ep.q_lo + ((size_t)gm * Hq + gh) * D;
          store_bf16x8(lo + 8 * c, la);
          store_bf16x8(lo + half + 8 * c, lb);
        }
        continue;
      }
      const int blk = blk_sh[r];
      if (blk < 0) continue;
      const int slot = pos_sh[r] & (HL_BLOCK_SIZE - 1);
      if (gh < Hq + Hkv) {
        hl_bf16* dst = ep.kpool + (((size_t)blk * Hkv + (gh - Hq)) * HL_BLOCK_SIZE + slot) * D;
        store_bf16x8(dst + 8 * c, a);
        store_bf16x8(dst + half + 8 * c, b);
      } else {
        hl_bf16* dst = ep.vpool + ((size_t)blk * Hkv + (gh - Hq - Hkv)) * D * HL_BLOCK_SIZE + slot;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dst[(8 * c + e) * HL_BLOCK_SIZE] = (hl_bf16)f2bf(a[e]);
          dst[(half + 8 * c + e) * HL_BLOCK_SIZE] = (hl_bf16)f2bf(b[e]);
        }
      }
    }
    return;
  }
  const hl_bf16* R = ep.residual;
  const int ldc = (EPI == HL_EPI_SWIGLU) ? half_n : N;
  const int n0 = nt * OUT_N;
  constexpr int CH_PER_ROW = OUT_N / 8;
  for (int q = tid; q < BM * CH_PER_ROW; q += kThreads) {
    const int row = q / CH_PER_ROW, ch = q % CH_PER_ROW;
    const int gm = m0 + row;
    if (gm >= M) continue;
    const float* v = st + row * OUT_N + ch * 8;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = v[e];
    if (EPI == HL_EPI_RESIDUAL) {
      u32x4 rr = *reinterpret_cast<const u32x4*>(R + (size_t)gm * ldc + n0 + ch * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] += bf_lo(rr[e]);
        o[2 * e + 1] += bf_hi(rr[e]);
      }
    }
    u32x4 outv;
#pragma unroll
    for (int e = 0; e < 4; ++e) outv[e] = pack_bf2(o[2 * e], o[2 * e + 1]);
    *reinterpret_cast<u32x4*>(C + (size_t)gm * ldc + n0 + ch * 8) = outv;
  }
}

}  // namespace

namespace hl {

size_t gemm_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return 0; }

template <int EPI>
static void set_smem_attr() {
  static bool done = false;
  if (!done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_nt_kernel<EPI>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSmemTotal);
    (void)hipGetLastError();
    done = true;
  }
}

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void*, size_t, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  const int mtiles = (m + BM - 1) / BM;
  const int ntiles = n / BN;
  const dim3 grid(mtiles * ntiles), block(kThreads);
  switch (epi.kind) {
    case HL_EPI_NONE:
      set_smem_attr<HL_EPI_NONE>();
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_NONE>, grid, block, kSmemTotal, st, a, w, c,
                         m, n, k, mtiles, epi);
      break;
    case HL_EPI_RESIDUAL:
      set_smem_attr<HL_EPI_RESIDUAL>();
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_RESIDUAL>, grid, block, kSmemTotal, st, a, w,
                         c, m, n, k, mtiles, epi);
      break;
    case HL_EPI_SWIGLU:
      set_smem_attr<HL_EPI_SWIGLU>();
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_SWIGLU>, grid, block, kSmemTotal, st, a, w,
                         c, m, n, k, mtiles, epi);
      break;
    default:
      set_smem_attr<kEpiRopeAppend>();
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<kEpiRopeAppend>, grid, block, kSmemTotal, st, a, w,
                         c, m, n, k, mtiles, epi);
      break;
  }
  return hipGetLastError();
}

}  // namespace hl
