// Token-batched linear layer: the choice of tile shape and schedule for each launch.
//
// Prompt-chunk rows and decode rows of the hybrid batch share every linear layer, so one GEMM
// over the whole token matrix reads each weight once for both phases ("ConfluxServe" summary,
// "Why can linear layers be batched but attention cannot?"). The token count is whatever the
// batch brings (a 1024-token chunk plus 16 decodes is 1040 rows), so a fixed tile wastes up to a
// whole row of tiles, and the round of tiles that does not fill the compute units wastes more;
// the chunked-prefill page names this tile-quantisation cliff ("Chunked prefill (stall-free
// batching), explained", tile quantisation). Every launch therefore picks its tile shape, and
// between one tile per workgroup and a stream-K run, by a cost model of the launch:
//
//   one tile per workgroup: t = k_steps * c(BM, BN) * (full rounds + partial round share)
//     where a partial round of r tiles on 256 compute units costs (0.84 + 0.16 r / 256) of a full
//     one (its tiles run with less contention);
//   stream-K: t = 1.39 * ceil(tiles * k_steps / 256) * c(BM, BN) + 0.05 us per MB of fp32 pieces
//     (one piece per run end plus one per split tile, written and read back by the fix-up; a run
//     that changes tiles loses cache locality, hence the 1.39);
//   tail split (any epilogue): the full rounds as above, then the r tiles left over (r at most
//     half the compute units) cut into S = min(256 / r, 4) K ranges: t = k_steps * c(BM, BN) *
//     full rounds + 1.36 * ceil(k_steps / S) * c(BM, BN) * (0.84 + 0.16 r S / 256) + 0.05 us per MB
//     of pieces + 11 us (split-K's constants: the fix-up pass and the pieces' round trip);
//   split-K into S ranges: t = f * ceil(k_steps / S) * c(BM, BN) * (rounds of tiles * S) + 0.05 us
//     per MB of pieces (S per tile) + 11 us (the fix-up pass and the pieces' round trip), with
//     f = 1.36 for the 128-wide tiles, fitted to every 128-wide tile x S in {2, 3, 4, 6, 8} on the
//     SwiGLU and QKV projections of the 8B and 70B shapes at 65..1040 rows (relative rms error
//     12 %). Plain and residual GEMMs may also split the 256-wide tiles, at f = 1.0 (their long
//     split runs go at the one-tile k-step rate: 0.95-1.06 measured on the 70B and 14B O and down
//     projections); against the previous picks that made the 17 changed layer GEMMs of a sweep
//     (8B / 14B / 70B, 128..4160 rows) 14 % faster in total, none more than 1 % slower. For SwiGLU
//     and the QKV projection the wide splits were slower (up to 22 %), so there only the
//     128-wide tiles split.
// Over a sweep of every tile x schedule on the QKV, O, gate/up and down projections of the 8B, 14B
// and 70B shapes at 128..4160 rows (2954 timings), the model's picks take 1.2 % longer in total
// than the best measured pick of each GEMM.
//
// c(BM, BN) is the time of one 64-deep k-step of a BM x BN tile with every compute unit busy,
// fitted, together with the other constants, to times of all shapes below on the layer GEMMs of
// the four large workloads on MI355X (relative rms error 11 %; over those sixteen GEMMs the
// model's picks take 0.7 % longer in total than the measured best pick of each).
#include <algorithm>

#include "gemm_core.h"

namespace {

struct TileCost {
  int bm, bn;
  float kstep_us;
  bool streamk;  // also considered as a stream-K run (and, if 128 wide, as split-K)
  bool swiglu_only = false;  // one tile per workgroup, SwiGLU epilogue only
};
constexpr TileCost kTiles[] = {
    {256, 256, 1.579f, true},  {224, 256, 1.473f, true},  {192, 256, 1.285f, true},
    {160, 256, 1.136f, true},  {128, 256, 0.960f, true},  {256, 128, 0.929f, false},
    {224, 128, 0.853f, false}, {160, 128, 0.631f, false}, {128, 128, 0.547f, false},
    {256, 192, 1.40f, false, true}, {128, 192, 0.87f, false, true},
};
constexpr int kCUs = kStreamKGrid;
constexpr float kPartialRound = 0.84f;
// Split and stream-K prices. SwiGLU and the QKV projection (whose fix-ups also rotate and route
// rows) keep the constants fitted on the 128-wide split tiles; plain and residual GEMMs use a set
// fitted to every tile x schedule (one tile, stream-K, split-K into 2..8, tail split into 2..4)
// of the 8B / 14B / 70B O and down projections at 128..4160 rows: their picks take 0.66 % longer
// in total than the best measured schedule of each of those 51 GEMMs (mean 1.1 %, worst 11 %),
// against ~2 % for the constants fitted before, which under-priced stream-K's short runs at a few
// hundred rows and over-priced the long split runs of the 256-wide tiles. Those timings had the
// weights warm in the last-level cache; inside a step they are cold (a layer's weights exceed that
// cache). The wide split factor is refitted on every tile x schedule of the 8B / 14B / 70B O and
// down projections at 128..4160 rows timed with the weight evicted before each launch (24 GEMMs):
// 1.0 leaves 0.23 % of their total over the best schedule of each, 0.92 1.5 %.
struct SchedCost {
  float split_step, split_step_wide, split_fixed, piece_us_per_mb, streamk_step, streamk_fixed;
};
constexpr SchedCost kCostEpilogue = {1.36f, 1.36f, 11.0f, 0.05f, 1.39f, 0.0f};
constexpr SchedCost kCostPlain = {0.9f, 1.0f, 3.0f, 0.08f, 1.1f, 5.0f};
constexpr int kSplitCandidates[] = {2, 3, 4, 6, 8, 12, 16};
constexpr int kMinSplitSteps = 4;  // k-steps of 64 per split at least

const SchedCost& sched_cost(bool plain) { return plain ? kCostPlain : kCostEpilogue; }

float rounds(long items) {
  const long full = items / kCUs, rem = items % kCUs;
  return (float)full + (rem ? kPartialRound + (1.f - kPartialRound) * (float)rem / kCUs : 0.f);
}

float one_tile_cost(const TileCost& t, int m, int n, int nk) {
  const long tiles = (long)((m + t.bm - 1) / t.bm) * (n / t.bn);
  return nk * t.kstep_us * rounds(tiles);
}

float split_step(const TileCost& t, bool plain) {
  const SchedCost& c = sched_cost(plain);
  return t.bn == 128 ? c.split_step : c.split_step_wide;
}

float split_cost(const TileCost& t, int m, int n, int nk, int s, bool plain) {
  const long tiles = (long)((m + t.bm - 1) / t.bm) * (n / t.bn);
  const float mb = (float)s * tiles * t.bm * t.bn * 8 / 1e6f;
  return (float)((nk + s - 1) / s) * t.kstep_us * rounds(tiles * s) * split_step(t, plain) +
         sched_cost(plain).piece_us_per_mb * mb + sched_cost(plain).split_fixed;
}

// one tile per workgroup with the last partial round split along K; S = 0 if not applicable
int tail_splits(const TileCost& t, int m, int n, int nk) {
  const long tiles = (long)((m + t.bm - 1) / t.bm) * (n / t.bn);
  const long rem = tiles % kCUs;
  if (tiles < kCUs || rem == 0 || 2 * rem > kCUs) return 0;
  const int s = (int)std::min<long>(4, kCUs / rem);
  if (nk < s * kMinSplitSteps || !tail_fits((int)rem, t.bm, t.bn, s)) return 0;
  return s;
}

float tail_cost(const TileCost& t, int m, int n, int nk, int s, bool plain) {
  const long tiles = (long)((m + t.bm - 1) / t.bm) * (n / t.bn);
  const long rem = tiles % kCUs, full = tiles / kCUs;
  const float mb = (float)s * rem * t.bm * t.bn * 8 / 1e6f;
  return nk * t.kstep_us * (float)full +
         (float)((nk + s - 1) / s) * t.kstep_us * split_step(t, plain) *
             (kPartialRound + (1.f - kPartialRound) * (float)(rem * s) / kCUs) +
         sched_cost(plain).piece_us_per_mb * mb + sched_cost(plain).split_fixed;
}

float streamk_cost(const TileCost& t, int m, int n, int nk) {
  const long tiles = (long)((m + t.bm - 1) / t.bm) * (n / t.bn);
  const long per = (tiles * nk + kCUs - 1) / kCUs;
  const long split = per < nk ? tiles : std::min<long>(tiles, kCUs);
  const long pieces = std::min<long>(2 * kCUs, kCUs + split);
  const float mb = (float)pieces * t.bm * t.bn * 8 / 1e6f;
  return per * t.kstep_us * kCostPlain.streamk_step + kCostPlain.piece_us_per_mb * mb +
         kCostPlain.streamk_fixed;
}

}  // namespace

namespace hl {

// Cheapest tile shape (and schedule) by the model above. `schedules`: kSchedStreamK (plain /
// residual epilogues) and / or kSchedSplitK (SwiGLU / RoPE) when a workspace is present.
// `col_align`: N-tile widths must be a multiple of it (the RoPE epilogue needs whole heads).
TileChoice choose_tiles(int m, int n, int k, int schedules, int col_align) {
  const int nk = k / BK;
  TileChoice best{128, 128, false};
  float best_t = 3.4e38f;
  const bool wide = (schedules & kSchedWideSplit) != 0;
  for (const TileCost& t : kTiles) {
    if (n % t.bn || t.bn % col_align) continue;
    const float c1 = one_tile_cost(t, m, n, nk);
    if (t.swiglu_only) {
      if ((schedules & kSchedSwigluTiles) && c1 < best_t) best_t = c1, best = TileChoice{t.bm, t.bn, false};
      continue;
    }
    if (c1 < best_t) best_t = c1, best = TileChoice{t.bm, t.bn, false};
    if (schedules & kSchedTail)
      if (const int s = tail_splits(t, m, n, nk)) {
        const float c4 = tail_cost(t, m, n, nk, s, wide);
        if (c4 < best_t) best_t = c4, best = TileChoice{t.bm, t.bn, false, s, true};
      }
    if ((schedules & kSchedStreamK) && t.streamk && nk >= 4) {
      const float c2 = streamk_cost(t, m, n, nk);
      if (c2 < best_t) best_t = c2, best = TileChoice{t.bm, t.bn, true};
    }
    if ((schedules & kSchedSplitK) && (t.bn == 128 || wide))
      for (int s : kSplitCandidates) {
        if (nk < s * kMinSplitSteps || !split_fits(m, n, t.bm, t.bn, s)) continue;
        const float c3 = split_cost(t, m, n, nk, s, wide);
        if (c3 < best_t) best_t = c3, best = TileChoice{t.bm, t.bn, false, s};
      }
  }
  return best;
}

bool use_skinny(int m, int n, int k, size_t ws_bytes) {
  return m > 0 && m <= kSkinnyMaxM && n % 64 == 0 && ws_bytes >= skinny_workspace_bytes(m, n, k);
}

bool gemm_split_fits(int m, int n, int bm, int bn, int splits) {
  return split_fits(m, n, bm, bn, splits);
}

bool gemm_tail_fits(int m, int n, int bm, int bn, int splits) {
  const int tiles = ((m + bm - 1) / bm) * (n / bn);
  return tail_fits(tiles - tail_full_tiles(tiles), bm, bn, splits);
}

bool gemm_tile_supported(int bm, int bn, int epilogue, int stream_k) {
  for (const TileCost& t : kTiles)
    if (t.bm == bm && t.bn == bn)
      return !t.swiglu_only || (epilogue == HL_EPI_SWIGLU && stream_k == 0);
  return false;
}

hipError_t launch_gemm_tiles(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                             int32_t k, const GemmEpi& epi, const TileChoice& tc, void* ws,
                             hipStream_t st) {
  float* part = static_cast<float*>(ws);
  switch (epi.kind) {
    case HL_EPI_NONE: return launch_gemm_plain(tc, a, w, c, m, n, k, epi, part, st);
    case HL_EPI_RESIDUAL: return launch_gemm_residual(tc, a, w, c, m, n, k, epi, part, st);
    default: return launch_gemm_swiglu(tc, a, w, c, m, n, k, epi, part, st);
  }
}

// Stream-K pieces: up to kStreamKGrid workgroups x 2 pieces x a 256 x 256 fp32 tile.
size_t gemm_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return kStreamKWorkspace; }

hipError_t launch_gemm(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, int32_t m, int32_t n,
                       int32_t k, const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  float* part = (ws && ws_bytes >= kStreamKWorkspace) ? static_cast<float*>(ws) : nullptr;
  // few tokens: stream the weights with every compute unit (split K), when the partials fit
  if (ws && use_skinny(m, n, k, ws_bytes))
    return launch_gemm_skinny(a, w, c, m, n, k, epi, static_cast<float*>(ws), st);
  switch (epi.kind) {
    case HL_EPI_NONE:
      return launch_gemm_plain(
          choose_tiles(m, n, k, part ? kSchedStreamK | kSchedSplitK | kSchedWideSplit | kSchedTail : 0,
                       1),
          a, w, c, m, n, k, epi, part, st);
    case HL_EPI_RESIDUAL:
      return launch_gemm_residual(
          choose_tiles(m, n, k, part ? kSchedStreamK | kSchedSplitK | kSchedWideSplit | kSchedTail : 0,
                       1),
          a, w, c, m, n, k, epi, part, st);
    case HL_EPI_SWIGLU:
      return launch_gemm_swiglu(
          choose_tiles(m, n, k, kSchedSwigluTiles | (part ? kSchedSplitK | kSchedTail : 0), 1), a,
          w, c, m, n, k, epi, part, st);
    default:
      return launch_gemm_rope(
          choose_tiles(m, n, k, part ? kSchedSplitK | kSchedTail : 0, epi.head_dim), a, w, c, m,
          n, k, epi, part, st);
  }
}

}  // namespace hl
