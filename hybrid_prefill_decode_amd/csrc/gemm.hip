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
// is fetched from HBM about once. Epilogues run on fp32 staged in LDS: plain, + residual, and
// SwiGLU (the 128-row W tile holds 64 gate rows and the matching 64 up rows).
#include "common.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64, kThreads = 256;
constexpr int kTileBytes = 128 * BK * 2;         // one 128 x 64 bf16 operand tile
constexpr int kStageBytes = 2 * kTileBytes;      // A + W
constexpr int kSmemBytes = 2 * kStageBytes;      // double buffered: 64 KB

HL_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Bijection from dispatch order to tile order that keeps consecutive tiles on one XCD.
HL_DEV int xcd_tile(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_nt_kernel(
    const hl_bf16* __restrict__ A, const hl_bf16* __restrict__ W, hl_bf16* __restrict__ C,
    const hl_bf16* __restrict__ R, int M, int N, int K, int mtiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
      if (EPI == HL_EPI_SWIGLU) {
        const float g = acc[i][0][r], u = acc[i][1][r];
        const float s = g / (1.f + __expf(-g));
        st[row * OUT_N + wn * 32 + (lane & 31)] = s * u;
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          st[row * OUT_N + wn * 64 + t * 32 + (lane & 31)] = acc[i][t][r];
      }
    }
  }
  __syncthreads();
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

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, const hl_bf16* res,
                       int32_t m, int32_t n, int32_t k, int32_t epi, void*, size_t,
                       hipStream_t st) {
  if (m <= 0) return hipSuccess;
  const int mtiles = (m + BM - 1) / BM;
  const int ntiles = n / BN;
  const dim3 grid(mtiles * ntiles), block(kThreads);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_nt_kernel<HL_EPI_NONE>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_nt_kernel<HL_EPI_RESIDUAL>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_nt_kernel<HL_EPI_SWIGLU>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    (void)hipGetLastError();
    attr_set = true;
  }
  switch (epi) {
    case HL_EPI_NONE:
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_NONE>, grid, block, kSmemBytes, st, a, w, c,
                         res, m, n, k, mtiles);
      break;
    case HL_EPI_RESIDUAL:
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_RESIDUAL>, grid, block, kSmemBytes, st, a,
                         w, c, res, m, n, k, mtiles);
      break;
    default:
      hipLaunchKernelGGL(gemm_bf16_nt_kernel<HL_EPI_SWIGLU>, grid, block, kSmemBytes, st, a, w,
                         c, res, m, n, k, mtiles);
      break;
  }
  return hipGetLastError();
}

}  // namespace hl
