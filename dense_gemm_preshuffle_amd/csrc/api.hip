// Host side of the preshuffle GEMM library: argument validation, the tile
// planner, the B preshuffle kernel and the exported C entry points.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gemm_preshuffle.h"
#include "launch.hpp"
#include "variants.hpp"

namespace gp {
namespace {

constexpr int64_t kMaxBytes = (int64_t)1 << 31;  // 32-bit buffer offsets

// rows * row_bytes < kMaxBytes, decided without forming the product (rows and
// row_bytes are positive; a product of two sizes near 2^62 would overflow)
bool fits(int64_t rows, int64_t row_bytes) { return row_bytes < kMaxBytes && rows <= (kMaxBytes - 1) / row_bytes; }

// Bits per element of B (and of A, except W4A8 whose A is int8).
int elem_bits(int dt) {
  switch (dt) {
    case GP_I8:
    case GP_FP8_E4M3: return 8;
    case GP_BF16:
    case GP_F16: return 16;
    case GP_FP4_E2M1:
    case GP_I4: return 4;
    default: return 0;
  }
}
int a_bits(int dt) { return dt == GP_I4 ? 8 : elem_bits(dt); }

// Kernel-side dtype tag of an input gp_dtype.
int kdt(int dt) {
  switch (dt) {
    case GP_I8: return DT_I8;
    case GP_FP8_E4M3: return DT_FP8;
    case GP_BF16: return DT_BF16;
    case GP_F16: return DT_F16;
    case GP_I4: return DT_I4;
    default: return DT_FP4;
  }
}

struct TileVar { int dt, ms, tm, tn, tkb, pipe, kg; };
struct SplitVar { int dt, nb, waves, kch, mb; };
struct WideVar { int dt, ms, tkb, pipe; };

#define GP_TILE_ENTRY(DT, MS, TM, TN, TKB, PIPE) {DT, MS, TM, TN, TKB, PIPE, 1},
#define GP_TILE_KG2_ENTRY(DT, MS, TM, TN, TKB, PIPE) {DT, MS, TM, TN, TKB, PIPE, 2},
#define GP_SPLIT_ENTRY(DT, NB, W, KCH, MB) {DT, NB, W, KCH, MB},
#define GP_WIDE_ENTRY(DT, MS, TKB, PIPE) {DT, MS, TKB, PIPE},
constexpr TileVar kTiles[] = {GP_TILE_ALL(GP_TILE_ENTRY) GP_TILE_KG2_ALL(GP_TILE_KG2_ENTRY)};
constexpr TileVar kNoSched[] = {GP_TILE_NOSCHED_ALL(GP_TILE_ENTRY)};
constexpr TileVar kKSplit[] = {GP_TILE_KSPLIT_ALL(GP_TILE_ENTRY)};
constexpr SplitVar kSplits[] = {GP_SPLITK_ALL(GP_SPLIT_ENTRY)};
constexpr WideVar kWides[] = {GP_WIDE_ALL(GP_WIDE_ENTRY)};

bool tile_compiled(int dt, int ms, int tm, int tn, int tkb, int pipe = -1, int kg = 1) {
  for (const auto& v : kTiles)
    if (v.dt == dt && v.ms == ms && v.tm == tm && v.tn == tn && v.tkb == tkb && (pipe < 0 || v.pipe == pipe) &&
        v.kg == kg)
      return true;
  return false;
}

// Pipeline for a compiled tile: the caller's (opts.pipeline 1 = VGPR-staged
// A, 2 .. 6 = LDS DMA with that many stages), else by the default order.
int pick_pipe(int dt, int ms, int tm, int tn, int tkb, int want) {
  if (want > 0) {
    const int pipe = want == 1 ? 0 : want;
    return tile_compiled(dt, ms, tm, tn, tkb, pipe) ? pipe : -1;
  }
  // FP4's 3-stage variant spills at 128x256; elsewhere the deepest wins
  const int order[3][3] = {{3, 2, 0}, {2, 3, 0}, {0, 0, 0}};
  const int* ord = dt == DT_FP4 ? order[1] : order[0];
  for (int k = 0; k < 3; ++k)
    if (tile_compiled(dt, ms, tm, tn, tkb, ord[k])) return ord[k];
  return -1;
}
// A variant with the compiler's own hot-loop order (scheduler off) exists.
bool nosched_compiled(int dt, int ms, int tm, int tn, int tkb, int pipe) {
  for (const auto& v : kNoSched)
    if (v.dt == dt && v.ms == ms && v.tm == tm && v.tn == tn && v.tkb == tkb && v.pipe == pipe) return true;
  return false;
}
// A variant able to split K across workgroups exists.
bool ksplit_compiled(int dt, int ms, int tm, int tn, int tkb, int pipe) {
  for (const auto& v : kKSplit)
    if (v.dt == dt && v.ms == ms && v.tm == tm && v.tn == tn && v.tkb == tkb && v.pipe == pipe) return true;
  return false;
}
bool split_compiled(int dt, int nb, int waves, int kch, int mb) {
  for (const auto& v : kSplits)
    if (v.dt == dt && v.nb == nb && v.waves == waves && v.kch == kch && v.mb == mb) return true;
  return false;
}

struct Plan {
  int kernel = 0;
  int ms = 16;                  // MFMA block (16 or 32)
  int pipe = 0;                 // 0 VGPR-staged A, 2 .. 6 LDS DMA stages
  int tm = 0, tn = 0, tkb = 0;  // tile and wide kernels (tkb in bytes)
  int kg = 1;                   // tile kernel: K groups of 4 waves
  int epi = EPI_DIRECT;
  int xcd = 1;
  int nb = 0, waves = 4, kch = 0, mb = 1;  // split-K kernel (mb: 16-row blocks per workgroup)
  int ks = 1;                   // tile kernel: K split across workgroups
  int sched = 1;                // tile kernel: 1 pinned hot-loop schedule, 2 the compiler's
  int64_t Kb = 0;
};

// Workspace of a K split across workgroups: a fixed area of arrival counters
// (4 bytes per tile, for up to kMaxSplitTiles tiles), then ks partial tiles of
// TM x TN 4-byte sums per tile. The counter area is the same for every
// shape, so a workspace whose counters are zero (as every call leaves them)
// can serve calls of any shape: a later call's counters never fall where an
// earlier call left partial sums.
constexpr int64_t kMaxSplitTiles = 16384;
constexpr int64_t kCounterBytes = kMaxSplitTiles * 4;
int64_t tiles_of(const Plan& p, int64_t M, int64_t N) { return ((M + p.tm - 1) / p.tm) * ((N + p.tn - 1) / p.tn); }
int64_t workspace_bytes(const Plan& p, int64_t M, int64_t N) {
  if (p.ks <= 1) return 0;
  return kCounterBytes + tiles_of(p, M, N) * p.ks * p.tm * p.tn * 4;
}

// K bytes of B one MFMA consumes (per MS x MS block); a W4A8 piece of 64
// B bytes feeds two int8 MFMAs
int kernel_mfma_kb(int dt, int ms) { return ms == 32 ? 32 : (dt == DT_FP8 ? 128 : dt == DT_I4 ? 32 : 64); }

// MFMA block for a tile: the caller's, else 32x32 for FP4 (measured faster
// on the MXFP4 4096x4096x8192 shape), else 16x16 where compiled. (BF16
// measures the same with either block at 128x256: its loop is bound by the
// operand loads, not by the MFMA issue rate.)
int pick_ms(int dt, int tm, int tn, int tkb, int want) {
  if (want == 16 || want == 32) return tile_compiled(dt, want, tm, tn, tkb) ? want : 0;
  const bool prefer32 = dt == DT_FP4;
  if (prefer32 && tile_compiled(dt, 32, tm, tn, tkb)) return 32;
  if (tile_compiled(dt, 16, tm, tn, tkb)) return 16;
  if (tile_compiled(dt, 32, tm, tn, tkb)) return 32;
  return 0;
}

// Default tile preference (largest first) per input type, tile_k in bytes.
// Named shapes: FP8 medium 64x256x128 (GEMM Optimization Guide §1.3), BF16
// large 128x256x64 elements, FP4 64-128 x 256 x 256 elements.
// Workgroups that count as a full grid for the planner's first choice:
// three quarters of the 256 CUs. With a stricter 256, 7168 columns (224
// tiles of 128 columns) sent FP8 256 x 7168 x 2048 to 16 x 64 tiles (1792
// workgroups, 19.1 us) instead of 64 x 128 ones (224 workgroups, 9.7 us).
constexpr int64_t kFullGrid = 192;

int choose_tile(int dt, int64_t M, int64_t N, int64_t Kb, Plan* p, int want_ms) {
  struct Cand { int tm, tn, tkb, min_grid = 0; };
  // (the 64-byte K tiles at the ends of the lists serve K not a multiple of
  // the larger ones: one 64-byte K block is the layout's granularity)
  static const Cand i8[] = {{128, 256, 128}, {64, 256, 128}, {64, 128, 256}, {64, 128, 128}, {128, 128, 128},
                            {64, 64, 128}, {32, 64, 128}, {16, 64, 256}, {128, 256, 64}, {64, 128, 64}};
  // FP8: in the order of operand bytes per FLOP (1/TM + 1/TN): 128 x 128
  // before 64 x 256 (1024 x 4096 x 7168 36.5 us against 39.8, 512 x 7168 x
  // 2048 13.8 against 14.6 on 64 x 128), 64 x 128 x 256 before 32 x 256 x
  // 256 (512 x 4096 x 4096 15.4 against 20.0 us), 32 x 128 before 16 x 64
  // (128 x 7168 x 2048 8.0 against 13.1).
  static const Cand fp8[] = {{128, 256, 128}, {128, 128, 256}, {128, 128, 128}, {64, 256, 128}, {64, 128, 256},
                             {32, 256, 256}, {32, 256, 128}, {64, 128, 128}, {32, 128, 256}, {16, 64, 512}};
  // BF16 / FP16: 256 x 256 on 8 waves (each wave 32 columns of all 256
  // rows, so a B byte a wave loads feeds 256 rows) where it gives at least
  // 256 tiles: BF16 8192^3 727-734 us against 757 for 128 x 512 on 8 waves,
  // 4096^3 100-101 against 109, 4096 x 8192 x 8192 371 against 390-392,
  // 16384 x 4096 x 4096 385-386 against 402-403, 8192 x 8192 x 2048 213-214
  // against 215-218; FP16 8192^3 766-767 against 786-788 (one process
  // each). Then 128 x 512 on 8 waves where it still gives at least 1024
  // tiles (8192^3 771.7 us against 783.0 for 128 x 256, before the 256 x
  // 256 form).
  static const Cand b16[] = {{256, 256, 128, 256}, {128, 512, 128, 1024}, {128, 256, 128}, {64, 256, 128},
                             {128, 128, 128}, {64, 128, 128}, {128, 256, 64}, {32, 128, 128}, {64, 128, 64}};
  // MXFP4: 128 x 512 on 8 waves where it gives a tile per CU: 4096 x 4096 x
  // 8192 69.7-70.0 us against 71.6-72.5 for 128 x 256 (one process; equal
  // with warm caches: the gain is in the bytes fetched)
  static const Cand fp4[] = {{128, 512, 128, 256}, {128, 256, 128}, {64, 256, 128}, {128, 128, 128},
                             {32, 256, 128}, {64, 128, 128}, {128, 256, 64}, {64, 128, 64}};
  // W4A8: tile_k in bytes of B (64 bytes = 128 INT4); A tiles twice as long
  static const Cand i4[] = {{128, 256, 64}, {64, 256, 64}, {64, 128, 128}, {64, 128, 64}, {32, 128, 64},
                            {32, 64, 64}};
  const Cand* list;
  int n;
  switch (dt) {
    case DT_I8: list = i8; n = sizeof(i8) / sizeof(Cand); break;
    case DT_FP8: list = fp8; n = sizeof(fp8) / sizeof(Cand); break;
    case DT_BF16:
    case DT_F16: list = b16; n = sizeof(b16) / sizeof(Cand); break;
    case DT_I4: list = i4; n = sizeof(i4) / sizeof(Cand); break;
    default: list = fp4; n = sizeof(fp4) / sizeof(Cand); break;
  }
  // Tile choice, all types but MXFP4: the tile whose busiest CU streams the
  // fewest operand bytes per byte of K, ceil(grid / 256) * (TM + TN), among
  // tiles whose edge tiles (overlapping their neighbours inside M x N) add at
  // most a quarter to the computed area; ties go to the earlier candidate.
  // Three corrections, each from a measured pair on one MI355X: divided by
  // 1.2 where a CU holds 8 waves or more (two resident workgroups, or one
  // 8-wave tile: more loads in flight; 1.35 made two 128 x 128 tiles per CU
  // beat one 128 x 256 on 1024 x 7168 x 2048, which measured 3-7% slower);
  // times (256 / grid)^0.3 where CUs stay idle; times 1.4 for tiles whose A
  // is staged through registers (BF16 64 x 128: 83 us against 59 with LDS
  // DMA on 256 x 8192 x 8192). This ranks the tiles of the FP8 / BF16 / FP16
  // / INT8 shapes timed for it (80 x 7168 x 2048 to 8192^3) in their
  // measured order, e.g. FP8 96 x 7168 x 2048 7.9 us on 168 tiles of 32 x 128
  // against 10.3 on 672 of 16 x 64 (the threshold rule's choice), BF16 768 x
  // 4096 x 4096 40.6 on 128 x 128 against 45.7 on 64 x 256, BF16 300 x 8192 x
  // 4096 45.4 on 320 tiles of 64 x 128 against 53.7 on 160 of 64 x 256.
  //
  // Threshold rule (MXFP4, whose 128 x 128 tile the count ranks wrongly:
  // 18.7 us against 17.0 for 64 x 256 on 512 x 7168 x 4096; and any type
  // when no tile passes the count's filters): the first tile in the list's
  // order that gives kFullGrid workgroups, else the one with the most.
  // Tiles whose grid covers at most 1/8 more than M x N come first, exact or
  // not, the rest only if none of those fits (preferring exact tiles
  // outright sent BF16 8000 x 8192 x 8192 to 64 x 256 tiles, 1616 us,
  // against 728 us on 256 x 256 tiles, 2.4% of whose rows are computed twice).
  if (dt != DT_FP4) {
    int best = -1;
    double best_cost = 0;
    for (int i = 0; i < n; ++i) {
      const Cand& c = list[i];
      if (c.tm > M || c.tn > N || Kb % c.tkb) continue;
      const int ms = pick_ms(dt, c.tm, c.tn, c.tkb, want_ms);
      if (!ms) continue;
      bool dma = false;
      for (int pipe = 2; pipe <= 6; ++pipe) dma = dma || tile_compiled(dt, ms, c.tm, c.tn, c.tkb, pipe);
      const int64_t gm = (M + c.tm - 1) / c.tm, gn = (N + c.tn - 1) / c.tn;
      if (gm * c.tm * gn * c.tn * 4 > M * N * 5) continue;
      const int64_t g = gm * gn;
      if (g < c.min_grid) continue;
      const int64_t rounds = (g + 255) / 256;
      // resident workgroups per CU: by registers, and by LDS (the A stages or
      // the CShuffle tile, whichever is larger)
      const int pipe = pick_pipe(dt, ms, c.tm, c.tn, c.tkb, 0);
      const int tka = c.tkb * (dt == DT_I4 ? 2 : 1);
      const int64_t lds = std::max<int64_t>((int64_t)(pipe > 2 ? pipe : 2) * c.tm * tka,
                                            c.tn >= 128 ? (int64_t)c.tm * (c.tn * (dt == DT_I8 ? 4 : 2) + 16) : 0);
      const int64_t wpc = std::max<int64_t>(1, std::min<int64_t>(tile_wgs_per_cu(c.tm, c.tn, 1), 160 * 1024 / lds));
      const int64_t waves = std::min<int64_t>(rounds, wpc) * tile_waves(c.tm, c.tn);
      double cost = (double)rounds * (c.tm + c.tn) * (dma ? 1.0 : 1.4) / (waves >= 8 ? 1.2 : 1.0);
      if (g < 256) cost *= std::pow(256.0 / (double)g, 0.3);
      if (best < 0 || cost < best_cost) { best = i; best_cost = cost; }
    }
    if (best >= 0) {
      p->tm = list[best].tm;
      p->tn = list[best].tn;
      p->tkb = list[best].tkb;
      p->ms = pick_ms(dt, p->tm, p->tn, p->tkb, want_ms);
      return GP_OK;
    }
  }
  for (int pass = 0; pass < 2; ++pass) {
    int best = -1;
    int64_t best_grid = -1;
    for (int i = 0; i < n; ++i) {
      const Cand& c = list[i];
      if (c.tm > M || c.tn > N || Kb % c.tkb) continue;
      const int64_t cover = ((M + c.tm - 1) / c.tm) * c.tm * (((N + c.tn - 1) / c.tn) * c.tn);
      const bool tight = cover * 8 <= M * N * 9;
      if (tight != (pass == 0)) continue;
      if (!pick_ms(dt, c.tm, c.tn, c.tkb, want_ms)) continue;
      const int64_t g = ((M + c.tm - 1) / c.tm) * ((N + c.tn - 1) / c.tn);
      if (g < c.min_grid) continue;
      if (g >= kFullGrid) { best = i; break; }
      if (g > best_grid) { best_grid = g; best = i; }
    }
    if (best >= 0) {
      p->tm = list[best].tm;
      p->tn = list[best].tn;
      p->tkb = list[best].tkb;
      p->ms = pick_ms(dt, p->tm, p->tn, p->tkb, want_ms);
      return GP_OK;
    }
  }
  return GP_ESHAPE;
}

// Compiled split-K chunk for (dt, nb, waves) that divides the wave's K range:
// the largest one up to 512 bytes (measured best for the M=16 FP8 shape),
// else the smallest; 0 if none.
int pick_chunk(int dt, int nb, int waves, int mb, int64_t kw) {
  int kch = 0;
  for (const auto& v : kSplits)
    if (v.dt == dt && v.nb == nb && v.waves == waves && v.mb == mb && kw % v.kch == 0 && v.kch <= 512 && v.kch > kch)
      kch = v.kch;
  if (kch == 0)
    for (const auto& v : kSplits)
      if (v.dt == dt && v.nb == nb && v.waves == waves && v.mb == mb && kw % v.kch == 0 && (kch == 0 || v.kch < kch))
        kch = v.kch;
  return kch;
}

// Bytes the busiest CU pulls for a small-M plan of mb 16-row and nb 16-column
// blocks per workgroup: its ceil(grid / 256) rounds of workgroups, each
// reading its B columns over the whole K and half of its A rows (A comes from
// L2, at about half the cost per byte on the M=16 shape).
double small_m_cost(int dt, int64_t M, int64_t N, int64_t Kb, int mb, int nb) {
  const int64_t Ka = Kb * (dt == DT_I4 ? 2 : 1), rows = std::min<int64_t>(M, 16 * mb);
  const int64_t grid = (N / (16 * nb)) * ((M + 16 * mb - 1) / (16 * mb));
  return (double)((grid + 255) / 256) * ((double)(16 * nb) * Kb + 0.5 * (double)rows * Ka);
}

int choose_split(int dt, int bits, int64_t M, int64_t N, int64_t Kb, Plan* p, const gemm_opts* o) {
  if (o && o->tile_n > 0 && o->tile_n % 16) return GP_ESHAPE;
  if (o && o->tile_m > 0 && o->tile_m != 16 && o->tile_m != 32 && o->tile_m != 64) return GP_ESHAPE;
  if (o && o->tile_k > 0 && ((int64_t)o->tile_k * bits) % 8) return GP_ESHAPE;
  const int user_kch = (o && o->tile_k > 0) ? (int)((int64_t)o->tile_k * bits / 8) : 0;
  // (waves, 16-row blocks per workgroup mb, 16-column blocks nb): the
  // caller's, else the compiled pair that leaves the busiest CU the fewest
  // bytes over its ceil(grid / 256) rounds of workgroups, counting B's bytes
  // and half of A's (read from L2; they cost about half as much per byte on
  // the M=16 shape), ties to more rows, then to two column blocks. More rows
  // per workgroup read B once for all of them but give fewer workgroups; four
  // blocks run on 8 waves, not for MXFP4 (7.2 us against 8.2 on two at
  // 64 x 7168 x 2048). One wave is the last resort (K too short for 4).
  // Measured (one MI355X; FP8 unless named; rows per workgroup):
  //   M=16, K=2048: N=2048 3.26 us on one column block (128 workgroups)
  //     against 3.81 on two, N=4096 3.64 against 3.99, N=5120 4.19 on two
  //     (160) against 4.97 on one (320), N=7168 4.44 on two (224);
  //   64 x 7168 x 2048: 7.4 on 64 rows, 8.4 on 32, 11.2 on 16;
  //   64 x 4096 x 4096: 7.8 on 32, 11.5 on 64, 10.5 on 16;
  //   64 x 2048 x 4096: 5.9 on 16, 7.5 on 32, 11.4 on 64; BF16 64 x 1024 x
  //   7168 13.6 on 16 against 33.9 on 64; 24 x 4096 x 2048 4.2 on 16, 4.9
  //   on 32. Over 288 shapes (six types, 24-64 rows, N 1024-7168, K
  //   2048-7168) this choice summed to 2628 us (with MXFP4's 128-byte
  //   chunks), against 3485 for 64 rows above 32 and 32 above 16.
  struct WM { int waves, mb; };
  WM cand[3];
  int nc = 0;
  if (o && o->tile_m > 0) {
    const int mb = o->tile_m / 16;
    cand[nc++] = {o->waves > 0 ? o->waves : (mb == 4 ? 8 : 4), mb};
  } else if (o && o->waves > 0) {
    if (M > 16) cand[nc++] = {o->waves, 2};
    cand[nc++] = {o->waves, 1};
  } else {
    if (M > 32 && dt != DT_FP4) cand[nc++] = {8, 4};
    if (M > 16) cand[nc++] = {4, 2};
    cand[nc++] = {4, 1};
  }
  int nbc[2] = {2, 1};
  int nn = 2;
  if (o && o->tile_n > 0) { nbc[0] = o->tile_n / 16; nn = 1; }
  // the chunk (K bytes per wave step) of one (waves, mb, nb), 0 if not compiled
  auto chunk = [&](int waves, int mb, int nb) {
    if (Kb % waves || N % (16 * nb)) return 0;
    const int64_t kw = Kb / waves;
    const int kch = user_kch ? user_kch : pick_chunk(dt, nb, waves, mb, kw);
    if (kch == 0 || kw % kch || !split_compiled(dt, nb, waves, kch, mb)) return 0;
    return kch;
  };
  double best = -1;
  for (int i = 0; i < nc; ++i) {
    const int waves = cand[i].waves, mb = cand[i].mb;
    for (int c = 0; c < nn; ++c) {
      const int nb = nbc[c];
      const int kch = chunk(waves, mb, nb);
      if (!kch) continue;
      const double cost = small_m_cost(dt, M, N, Kb, mb, nb);
      if (best >= 0 && cost >= best) continue;
      best = cost;
      p->nb = nb;
      p->waves = waves;
      p->kch = kch;
      p->mb = mb;
    }
  }
  if (best >= 0) return GP_OK;
  if (!(o && (o->tile_m > 0 || o->waves > 0))) {
    for (int c = 0; c < nn; ++c) {
      const int kch = chunk(1, 1, nbc[c]);
      if (!kch) continue;
      p->nb = nbc[c];
      p->waves = 1;
      p->kch = kch;
      p->mb = 1;
      return GP_OK;
    }
  }
  return GP_ESHAPE;
}

// K split across workgroups chosen by the planner (calls with a workspace):
// only where the tiles alone leave the GPU short of work, i.e. fewer than
// 256 workgroups, or 256 only with a tile smaller than 64 x 128 (each CU then
// pulls more operand bytes per FLOP from L2). The first tile (in the order
// of the split variants' list) takes the fewest ranges S (powers of two, up
// to 16, each range keeping at least 2048 K elements) that give 256
// workgroups, or the most such ranges if those give at least 128 (128 large
// tiles measured faster than 256 small ones on BF16), adjusted per type
// (in the function). A split costs a round
// trip of the partial sums at the end of the kernel (a few microseconds), so
// short K stays unsplit: FP8 512 x 4096 x 4096 measured 15.6 us unsplit and
// 20.0 us split in two; FP8 256 x 2048 x 16384 39.0 us unsplit (16 x 64
// tiles) and 20.8 us split in four (64 x 128 tiles); BF16 512 x 2048 x 16384
// 141.8 and 56.5 us (128 x 256 tiles, eight ranges); MXFP4 256 x 4096 x
// 16384 43.8 and 23.7 us (128 x 128 tiles, four ranges).
// Long K on a full grid of small tiles: where a split tile pulls fewer
// operand bytes per FLOP than the planner's tile (1/TM + 1/TN smaller), its
// first S (power of two) that gives 256 to 512 workgroups while each range
// keeps at least 4096 bytes of B's K: BF16 512 x 8192 x 8192 70 us on
// 128 x 256 tiles split in two against 88 on 64 x 256 tiles, 256 x 8192 x
// 8192 53 us split in four against 59 on 64 x 128, 384 x 8192 x 8192 80
// against 90; FP16 512 x 8192 x 8192 71 against 87-89. BF16 / FP16 only:
// the same rule measured slower for FP8 (512 x 8192 x 8192 49 us on 128 x
// 128 tiles split in two against 46; 256 x 8192 x 8192 34 against 29) and
// INT8 (512 x 8192 x 8192 50.5 against 48.8), whose partial sums cost as
// much per tile for half the bytes of K.
// num / den: the most area the split tile's grid may cover, relative to M x N
bool ksplit_larger_tile(int dt, int64_t M, int64_t N, int64_t Kb, Plan* p, int num = 9, int den = 8) {
  // From 128-row tiles only while the split keeps one workgroup per CU: BF16
  // 512 x 8192 x 8192 69 us on 128 x 256 tiles split in two against 78 on
  // 128 x 128, but 2048 x 4096 x 4096 71 us split in two (512 workgroups)
  // against 59 unsplit on 128 x 256.
  if (dt != DT_BF16 && dt != DT_F16) return false;
  const int64_t max_wg = p->tm < 128 ? 512 : 256;
  const double bpf = 1.0 / p->tm + 1.0 / p->tn;
  for (int i = 0; i < (int)(sizeof(kKSplit) / sizeof(kKSplit[0])); ++i) {
    const TileVar& v = kKSplit[i];
    if (v.dt != dt || v.tm > M || v.tn > N || Kb % v.tkb) continue;
    if (1.0 / v.tm + 1.0 / v.tn >= bpf) continue;
    const int64_t T = ((M + v.tm - 1) / v.tm) * ((N + v.tn - 1) / v.tn);
    const int64_t cover = ((M + v.tm - 1) / v.tm) * v.tm * (((N + v.tn - 1) / v.tn) * v.tn);
    if (cover * den > M * N * num) continue;   // edge tiles computing too much extra
    const int64_t KT = Kb / v.tkb;
    for (int S = 2; S <= 16; S *= 2) {
      if (KT % S || Kb / S < 4096) break;
      if (T * S < 256) continue;
      if (T * S > max_wg) break;
      p->tm = v.tm;
      p->tn = v.tn;
      p->tkb = v.tkb;
      p->ms = v.ms;
      p->pipe = v.pipe;
      p->ks = S;
      return true;
    }
  }
  return false;
}

void auto_ksplit(int dt, int64_t M, int64_t N, int64_t Kb, Plan* p) {
  const int64_t grid0 = ((M + p->tm - 1) / p->tm) * ((N + p->tn - 1) / p->tn);
  if (grid0 >= 256 && p->tm * p->tn >= 64 * 128) {
    ksplit_larger_tile(dt, M, N, Kb, p);
    return;
  }
  // 192 .. 255 workgroups: only the BF16 / FP16 split onto a larger tile,
  // whose edge tiles may then cover up to a third more (BF16 192 x 8192 x
  // 8192: 52 us on 128 x 256 tiles split in four against 58 on 64 x 128;
  // FP8 256 x 7168 x 8192 measured 27.9 us unsplit against 32.5 with its
  // 64 x 128 tiles split in two)
  if (grid0 >= kFullGrid && p->tm * p->tn >= 64 * 128) {
    ksplit_larger_tile(dt, M, N, Kb, p, 4, 3);
    return;
  }
  // Otherwise the first split tile (in the list's order) that reaches at
  // least 128 workgroups, in the fewest power-of-two ranges S that reach 256,
  // each range holding at least 2048 K elements (2048 bytes of B, 1024 of
  // 4-bit B: MXFP4 384 x 2048 x 8192 16.2 us in four ranges against 23.8
  // unsplit on 32 x 256 tiles, W4A8 128 x 7168 x 4096 11.6 in two against
  // 14.2). Adjustments by type, each measured on one MI355X:
  // - BF16 / FP16 skip their 128 x 256 tile while fewer than 32 of them
  //   cover the output, for 64 x 128 (128 x 2048 x 16384 32.4 us in eight
  //   ranges against 54.0 on 128 x 256 in eight, 384 x 2048 x 16384 52.2 in
  //   four against 83.9; from 32 the large tile held its own: 256 x 4096 x
  //   16384 62.0 against 63.3, 384 x 4096 x 8192 43.5 against 49.8); from 64
  //   of the small tiles they take twice the ranges, up to 512 workgroups
  //   (256 x 4096 x 8192 37.2 in four against 46.4 in two, 128 x 4096 x 8192
  //   28.4 in eight against 29.9 in four); and they leave 64 x 128 below 144
  //   workgroups for 16 x 64 tiles in more (FP16 80 x 512 x 16384 15.9 on
  //   320 against 23.1 on 128, 256 x 1024 x 7168 21.5 on 512 against 24.9).
  // - FP8 / INT8 on 64 x 128: four ranges where 48 to 64 tiles cover the
  //   output, from 4096 bytes of K and with the 64-row tiles covering at
  //   most 1.5 M (FP8 128 x 3072 x 4096 10.6 us against 12.7 on 16 x 64
  //   tiles in two, 256 x 2048 x 7168 13.7 against 16.5; INT8 192 x 2048 x
  //   4096 10.5 against 11.4; but FP8 80 x 3072 x 4096 10.5 against 9.4).
  // - FP8 / INT8 on 64 x 128 and MXFP4 / W4A8 on 64- and 128-row tiles: no
  //   more than 256 workgroups where halving S keeps at least 168 of them
  //   (FP8 160 x 4096 x 8192 18.7 us on 192 against 22.4 on 384, 384 x 7168
  //   x 4096 unsplit 21.5 against 26.0 on 672; INT8 384 x 1024 x 16384 19.5
  //   on 192 against 23.2 on 384; MXFP4 192 x 3072 x 16384 22.4 against
  //   29.5; W4A8 128 x 7168 x 8192 16.8 on 224 against 19.8 on 448), not
  //   below 168 (FP8 384 x 3072 x 16384 41.4 us on 288 against 48.4 on 144)
  //   and not below two ranges past 8192 K elements (FP8 160 x 7168 x 16384
  //   50.9 us in two against 52.7 unsplit; W4A8 192 x 7168 x 16384 34.9
  //   against 41.8). Not on 16 x 64 tiles, whose splits into 320-384
  //   workgroups beat half as many (FP8 192 x 1024 x 7168 11.0 against 12.2).
  const int64_t min_kb = (dt == DT_FP4 || dt == DT_I4) ? 1024 : 2048;
  int best = -1, best_s = 0;
  for (int i = 0; i < (int)(sizeof(kKSplit) / sizeof(kKSplit[0])); ++i) {
    const TileVar& v = kKSplit[i];
    if (v.dt != dt || v.tm > M || v.tn > N || Kb % v.tkb) continue;
    const bool half = dt == DT_BF16 || dt == DT_F16;
    if (half && v.tm == 128 && v.tn == 256 && ((M + 127) / 128) * ((N + 255) / 256) < 32) continue;
    const int64_t T = ((M + v.tm - 1) / v.tm) * ((N + v.tn - 1) / v.tn);
    const int64_t KT = Kb / v.tkb;
    int s_pick = 0;
    for (int S = 2; S <= 16; S *= 2) {
      if (KT % S || Kb / S < min_kb) break;
      s_pick = S;
      if (T * S >= 256) break;
    }
    if (half && v.tm == 64 && v.tn == 128 && T >= 64 && s_pick && T * s_pick <= 256 && T * s_pick * 2 <= 512 &&
        KT % (s_pick * 2) == 0 && Kb / (s_pick * 2) >= 2048)
      s_pick *= 2;
    const bool byte_tile = (dt == DT_FP8 || dt == DT_I8) && v.tm == 64 && v.tn == 128;
    if (byte_tile) {
      const bool rows_fit = ((M + 63) / 64) * 64 * 2 <= M * 3;   // the 64-row tiles cover at most 1.5 M
      if (T >= 48 && T <= 64 && rows_fit && Kb >= 4096 && KT % 4 == 0 && s_pick < 4) s_pick = 4;
    }
    if (byte_tile || ((dt == DT_FP4 || dt == DT_I4) && v.tm >= 64)) {
      const int64_t k_elems = (dt == DT_FP4 || dt == DT_I4) ? 2 * Kb : Kb;
      const int s_min = k_elems > 8192 ? 2 : 1;
      while (s_pick > s_min && T * s_pick > 256 && T * (s_pick / 2) >= 168) s_pick /= 2;
      if (s_pick == 1) return;   // the unsplit plan
    }
    if (!s_pick || T * s_pick < (half && v.tm == 64 && v.tn == 128 ? 144 : 128)) continue;
    best = i;
    best_s = s_pick;
    break;
  }
  if (best < 0) return;
  const TileVar& v = kKSplit[best];
  p->tm = v.tm;
  p->tn = v.tn;
  p->tkb = v.tkb;
  p->ms = v.ms;
  p->pipe = v.pipe;
  p->ks = best_s;
}

// Wide kernel (256x256 tiles, 8 waves, A and B through LDS): the caller's
// MFMA block (default 16), tile_k and pipeline where given; otherwise the
// compiled variant with the largest tile_k dividing K, then the most stages.
int choose_wide(int dt, int bits, int64_t M, int64_t N, int64_t Kb, Plan* p, const gemm_opts* o) {
  if (o && ((o->tile_m && o->tile_m != 256) || (o->tile_n && o->tile_n != 256))) return GP_ESHAPE;
  if (o && o->waves && o->waves != 8) return GP_ESHAPE;
  if (o && o->pipeline == 1) return GP_ESHAPE;   // both operands always go by LDS DMA
  if (M < 256 || N < 256) return GP_ESHAPE;   // edge tiles overlap inside M x N
  const int ms = (o && o->mfma) ? o->mfma : 16;
  int want_tkb = 0;
  if (o && o->tile_k) {
    if (((int64_t)o->tile_k * bits) % 8) return GP_ESHAPE;
    want_tkb = (int)((int64_t)o->tile_k * bits / 8);
  }
  const int want_pipe = o ? o->pipeline : 0;
  int best = -1;
  for (int i = 0; i < (int)(sizeof(kWides) / sizeof(kWides[0])); ++i) {
    const WideVar& v = kWides[i];
    if (v.dt != dt || v.ms != ms || Kb % v.tkb) continue;
    if ((want_tkb && v.tkb != want_tkb) || (want_pipe && v.pipe != want_pipe)) continue;
    if (best < 0 || v.tkb > kWides[best].tkb || (v.tkb == kWides[best].tkb && v.pipe > kWides[best].pipe)) best = i;
  }
  if (best < 0) return GP_ESHAPE;
  p->tm = p->tn = 256;
  p->ms = ms;
  p->tkb = kWides[best].tkb;
  p->pipe = kWides[best].pipe;
  p->epi = dt == DT_I8 ? EPI_DIRECT : EPI_CSHUFFLE;   // an int32 C tile does not fit LDS
  if (o && o->epilogue && o->epilogue != p->epi) return GP_ESHAPE;
  p->xcd = (o && o->xcd_swizzle) ? o->xcd_swizzle : 1;
  return GP_OK;
}

// 16 to 64 rows and long K, called with a workspace: 16 x 64 tiles (A
// through registers) whose K tiles are split across workgroups, in place of
// the small-M plan sm (null if that kernel cannot take the shape). S is the
// largest power of two that keeps at least 2048 bytes of B's K per range and
// at most 256 workgroups; taken where B's rows hold at least 8192 bytes (FP8)
// or 16384 (INT8, BF16, FP16, W4A8), S is 4 or more at 16 rows (2 or more
// above), and the busiest CU's bytes on the split (counted as for the
// small-M kernel) are at most a fraction of the small-M plan's: 0.8 (FP8
// from 16384 bytes of K: 0.95), W4A8 0.5. The small-M kernel streams more
// bytes per second per CU than the split tiles, whose partial sums and last
// arrivals cost too, so the split wins only where it cuts the bytes by that
// much: where the small-M plan takes one column block per workgroup (its A
// read once per 16 columns, ratio 0.38-0.75 here), not two (0.9; 0.83 for
// W4A8). Measured (one MI355X, graph replay, rotating inputs; small-M ->
// split): FP8 16 x 2048 x 16384 15.9 -> 11.5 us, 16 x 1024 x 32768 28.4 ->
// 14.9, 64 x 1024 x 16384 15.6 -> 11.2, 33 x 2048 x 32768 (ratio 0.9) 33.5
// -> 27.9 but 33 x 2048 x 8192 9.6 -> 10.1 (so not taken); INT8 24 x 1024 x
// 32768 26.0 -> 15.6, 33 x 2048 x 16384 16.9 -> 22.1 (ratio 0.9, not
// taken); BF16 16 x 1024 x 16384 27.3 -> 15.2, 64 x 2048 x 8192 16.3 ->
// 22.2 (not taken); W4A8 16 x 1024 x 65536 35.7 -> 19.6 (ratio 0.16), 33 x
// 1024 x 32768 19.0 -> 23.4 (0.62, not taken). Below those K the split lost
// at 16 rows (FP8 16 x 2048 x 7168 8.8 against 8.2, INT8 16 x 2048 x 8192
// 9.3 against 8.6, BF16 16 x 2048 x 4096 9.4 against 8.8, W4A8 16 x 2048 x
// 16384 11.2 against 10.8).
bool small_m_long_k(int dt, int64_t M, int64_t N, int64_t Kb, const Plan* sm, Plan* p) {
  if (M < 16 || M > 64 || N < 64 || dt == DT_FP4) return false;
  const int tkb = dt == DT_FP8 ? 512 : dt == DT_I4 ? 128 : 256;   // 512 bytes of A per K tile (W4A8: 256)
  if (Kb < (dt == DT_FP8 ? 8192 : 16384) || Kb % tkb) return false;
  if (!ksplit_compiled(dt, 16, 16, 64, tkb, 0)) return false;
  const int64_t T = ((M + 15) / 16) * ((N + 63) / 64), KT = Kb / tkb;
  int S = 0;
  for (int s = 2; s <= 64; s *= 2) {
    if (KT % s || Kb / s < 2048 || T * s > 256) break;
    S = s;
  }
  if (S < (M <= 16 ? 4 : 2)) return false;
  if (sm) {
    const int64_t Ka = Kb * (dt == DT_I4 ? 2 : 1);
    const double split = (double)((T * S + 255) / 256) * (double)(64 * Kb + 8 * Ka) / S;
    const double bound = dt == DT_I4 ? 0.5 : (dt == DT_FP8 && Kb >= 16384) ? 0.95 : 0.8;
    if (split > bound * small_m_cost(dt, M, N, Kb, sm->mb, sm->nb)) return false;
  }
  p->kernel = GP_KERNEL_TILE;
  p->ms = 16;
  p->tm = 16;
  p->tn = 64;
  p->tkb = tkb;
  p->pipe = 0;
  p->kg = 1;
  p->ks = S;
  p->sched = 1;
  p->epi = EPI_DIRECT;
  p->xcd = 1;
  return true;
}

// Above 64 rows the small-M kernel still beats the tile planner where the
// output is small: its workgroups re-read B once per 64 rows but stream it
// at a higher rate per CU, while the tiles of a small output leave CUs idle
// or split K at a cost. A rule per type on M x N and M x N x K, fitted to 216
// shapes per type (M 80-512, N 512-7168, K 1024-7168; one MI355X, graph
// replay, gemm_ex_ws plans on both sides; held-out halves of the shapes kept
// 97-100% of the better kernel's gain) and checked on 130 more (N 128-512 up
// to M = 4096, K up to 16384, M = 65 and 72). Summed over the 216, tile
// planner -> with the rule (the better kernel per shape): W4A8 3257 -> 2120
// (2120) us, MXFP4 2589 -> 2221 (2213), INT8 2483 -> 2279 (2264), BF16 4122
// -> 3873 (3836), FP16 4376 -> 4160 (4106), FP8 2211 -> 2176 (2160); e.g.
// W4A8 128 x 1024 x 7168 22.9 -> 4.9 us, BF16 128 x 2048 x 4096 17.0 ->
// 12.5, INT8 128 x 1024 x 4096 8.5 -> 5.5, W4A8 2048 x 256 x 7168 1.8x.
// Past 8192 columns of K the tiles' own K split wins for FP8, BF16, FP16 and
// INT8 (FP8 128 x 512 x 16384 11.0 us on split tiles against 15.3); for W4A8
// and MXFP4 (whose splits take ranges of 2048 K elements) from M x N x K =
// 2^31 (MXFP4 128 x 4096 x 8192 15.6 us in four ranges of 128 x 128 tiles
// against 24.9, but 128 x 1024 x 16384 on the small-M kernel 2.5x faster
// than split tiles; W4A8 128 x 4096 x 16384 18.6 against 33.4); below 1024
// the two are within the noise of a 3 us launch for INT8 and FP8, while
// BF16 / FP16 at K = 512-768 lose on the few tiles of a small output (BF16
// 111 x 256 x 512 3.0 us on the small-M kernel against 5.6 on 8 tiles,
// FP16 136 x 896 x 768 5.0 against 7.3).
// ws: a workspace is at hand, so the tiles may split K (without one the K
// bounds do not apply: unsplit tiles lose further, e.g. W4A8 384 x 1024 x 7168
// 34.9 us on 192 unsplit 32 x 64 tiles against 17.6 on the small-M kernel).
bool small_m_above_64(int dt, int64_t M, int64_t N, int64_t K, bool ws) {
  if (M <= 64 || M > 4096 || K < ((dt == DT_BF16 || dt == DT_F16) ? 512 : 1024)) return false;
  const double mn = (double)M * N, mnk = mn * (double)K;
  if (dt == DT_I4 || dt == DT_FP4) return mn <= (double)(1 << 19) && (!ws || mnk <= 2.0 * (double)(1 << 30));
  if (ws && K > 8192) return false;
  switch (dt) {
    case DT_I8: return mn <= (double)(3 << 18) && mnk <= 3.0 * (double)(1 << 29);
    case DT_BF16:
    case DT_F16: return mn <= (double)(3 << 18) && mnk <= (double)(1 << 30);
    default: return mn <= (double)(1 << 17) && mnk <= (double)(1 << 30);   // FP8
  }
}

// no option set: the planner chooses everything
bool no_options(const gemm_opts* o) {
  return !o || !(o->tile_m || o->tile_n || o->tile_k || o->epilogue || o->kernel || o->xcd_swizzle || o->waves ||
                 o->mfma || o->pipeline || o->ksplit || o->scheduler);
}

// ws: the call brings a workspace (gemm_ex_ws), so the tile kernel may split
// K across workgroups.
int make_plan(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* o, Plan* p, bool ws = false) {
  if (M <= 0 || N <= 0 || K <= 0) return GP_EINVAL;
  const int bits = elem_bits(in_dtype);
  if (bits == 0) return GP_EDTYPE;
  // every buffer is under 2^31 bytes, so no single size reaches it either;
  // rejected first, so that no product below can overflow
  if (M >= kMaxBytes || N >= kMaxBytes || K >= kMaxBytes) return GP_ESHAPE;
  if (o) {
    if (o->tile_m < 0 || o->tile_n < 0 || o->tile_k < 0 || o->waves < 0) return GP_EINVAL;
    if (o->epilogue < 0 || o->epilogue > 2 || o->kernel < 0 || o->kernel > 3) return GP_EINVAL;
    if (o->xcd_swizzle < 0 || o->xcd_swizzle > 2) return GP_EINVAL;
    if (o->mfma != 0 && o->mfma != 16 && o->mfma != 32) return GP_EINVAL;
    if (o->pipeline < 0 || o->pipeline > 6) return GP_EINVAL;
    if (o->ksplit < 0 || o->ksplit > 64) return GP_EINVAL;
    if (o->scheduler < 0 || o->scheduler > 2) return GP_EINVAL;
    if (o->ksplit > 1 && !ws) return GP_EWORKSPACE;   // a K split needs gemm_ex_ws
  }
  if ((K * bits) % 8) return GP_ESHAPE;
  const int64_t Kb = K * bits / 8;
  const int64_t Ka = K * a_bits(in_dtype) / 8;
  if (N % 16 || Kb % 64) return GP_ESHAPE;
  if ((in_dtype == GP_FP4_E2M1 || in_dtype == GP_I4) && K % 128) return GP_ESHAPE;
  if (in_dtype == GP_FP8_E4M3 && K % 128) return GP_ESHAPE;   // whole 16x16x128 MFMA steps
  // W4A8 accumulates 16 x the products in int32 (|a| <= 128, |b| <= 8)
  if (in_dtype == GP_I4 && K > 65536) return GP_ESHAPE;
  const int ob = in_dtype == GP_I8 ? 4 : 2;
  if (!fits(M, Ka) || !fits(N, Kb) || !fits(M, N * ob)) return GP_ESHAPE;
  const int dt = kdt(in_dtype);
  p->Kb = Kb;
  // small M (up to 64 rows): the split-K kernel; on 64 x 7168 x 2048 it
  // measured FP8 7.7 vs 8.1 us on tiles, INT8 7.1 vs 7.9, BF16 11.8 vs 20.8,
  // MXFP4 7.2 vs 9.4, W4A8 7.3 vs 11.9; at M = 128 on that N the tiles are as
  // fast or faster (FP8 12.7 vs 13.2). Above 64 rows, small outputs.
  const int64_t small_m = 64;
  const bool small_above = no_options(o) && small_m_above_64(dt, M, N, K, ws);
  p->kernel = (o && o->kernel) ? o->kernel : (M <= small_m || small_above ? GP_KERNEL_SPLITK : GP_KERNEL_TILE);
  if (dt == DT_I4 && p->kernel == GP_KERNEL_WIDE) return GP_EDTYPE;   // no 256 x 256 W4A8 kernel
  // a K split and the scheduler-off variants exist on the tile kernel only
  if (o && (o->ksplit > 1 || o->scheduler == 2) && p->kernel != GP_KERNEL_TILE) return GP_ESHAPE;
  if (p->kernel == GP_KERNEL_SPLITK) {
    Plan sm = *p;
    const int rc = choose_split(dt, bits, M, N, Kb, &sm, o);
    if (no_options(o) && ws && small_m_long_k(dt, M, N, Kb, rc == GP_OK ? &sm : nullptr, p)) return GP_OK;
    // FP8 on one wave per workgroup (its 128-byte MFMA steps do not split
    // evenly over more): the tiles, where one fits (32 x 576 x 4352 13.5 us
    // on the small-M kernel's single waves against 9.1 on five 32 x 128
    // tiles). Not the 4-bit types, whose single waves beat the tiles (W4A8
    // 511 x 576 x 11520 33.4 us against 54.1, MXFP4 39 x 6528 x 7936 23.6
    // against 26.4), nor 64-byte chunks on many workgroups (INT8 24 x 384 x
    // 12544 14.8 us on 48 workgroups of them against 28.8 on 12 tiles).
    const bool one_wave = rc == GP_OK && sm.waves == 1 && dt == DT_FP8 && no_options(o) && M >= 16 && N >= 64;
    if ((rc == GP_OK && !one_wave) || (rc != GP_OK && !small_above)) {
      *p = sm;
      return rc;
    }
    p->kernel = GP_KERNEL_TILE;   // the tile planner's choice (the small-M plan again if no tile fits)
  }
  if (p->kernel == GP_KERNEL_WIDE) return choose_wide(dt, bits, M, N, Kb, p, o);

  const bool user_tile = o && (o->tile_m || o->tile_n || o->tile_k);
  if (user_tile) {
    if (!(o->tile_m && o->tile_n && o->tile_k)) return GP_EINVAL;
    if (((int64_t)o->tile_k * bits) % 8) return GP_ESHAPE;
    p->tm = o->tile_m;
    p->tn = o->tile_n;
    p->tkb = (int)((int64_t)o->tile_k * bits / 8);
    p->ms = pick_ms(dt, p->tm, p->tn, p->tkb, o->mfma);
    if (!p->ms) return GP_ESHAPE;
    p->pipe = pick_pipe(dt, p->ms, p->tm, p->tn, p->tkb, o->pipeline);
    if (p->pipe < 0) return GP_ESHAPE;
    if (M < p->tm || N < p->tn || Kb % p->tkb) return GP_ESHAPE;
  } else {
    int r = choose_tile(dt, M, N, Kb, p, o ? o->mfma : 0);
    if (r) {
      // no tile fits inside M x N: the small-M kernel takes any M
      if (o && o->kernel == GP_KERNEL_TILE) return r;
      if (o && (o->ksplit > 1 || o->scheduler == 2)) return GP_ESHAPE;
      p->kernel = GP_KERNEL_SPLITK;
      return choose_split(dt, bits, M, N, Kb, p, o);
    }
    p->pipe = pick_pipe(dt, p->ms, p->tm, p->tn, p->tkb, o ? o->pipeline : 0);
    if (p->pipe < 0) return GP_ESHAPE;
  }
  // K groups: 8 waves asked for (two groups of 4 splitting the K tiles)
  if (o && o->waves && o->waves != 4) {
    // the caller left the pipeline to the planner: the one whose two-group form is compiled
    if (!o->pipeline && !tile_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe, 2))
      for (const auto& v : kTiles)
        if (v.kg == 2 && v.dt == dt && v.ms == p->ms && v.tm == p->tm && v.tn == p->tn && v.tkb == p->tkb) {
          p->pipe = v.pipe;
          break;
        }
    if (o->waves != 8 || (Kb / p->tkb) % 2 || !tile_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe, 2))
      return GP_ESHAPE;
    p->kg = 2;
  }
  // K split across workgroups: ksplit equal ranges of whole K tiles (of
  // whole K-group halves with two K groups)
  if (o && o->ksplit > 1) {
    if ((Kb / p->tkb) % ((int64_t)o->ksplit * p->kg)) return GP_ESHAPE;
    // the caller left the pipeline to the planner: the one whose split form is compiled
    if (!o->pipeline && !ksplit_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe))
      for (const auto& v : kKSplit)
        if (v.dt == dt && v.ms == p->ms && v.tm == p->tm && v.tn == p->tn && v.tkb == p->tkb) { p->pipe = v.pipe; break; }
    if (p->kg != 1 || !ksplit_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe)) return GP_ESHAPE;
    if (tiles_of(*p, M, N) > kMaxSplitTiles) return GP_ESHAPE;
    p->ks = o->ksplit;
  } else if (ws && !user_tile && p->kg == 1 && !(o && (o->ksplit == 1 || o->pipeline || o->mfma || o->scheduler))) {
    auto_ksplit(dt, M, N, Kb, p);
  }
  // W4A8 / MXFP4 past the M x N x K bound of the small-M rule but on fewer
  // than 128 workgroups of split tiles, or 256 unsplit ones (no split tile
  // fits, e.g. MXFP4 below 128 rows): the small-M kernel (MXFP4 96 x 2048 x
  // 16384 24.5 us against 44.4 on 24 unsplit 32 x 256 tiles, W4A8 511 x 576
  // x 11520 33.4 against 54.1 on 144 unsplit 32 x 64 tiles)
  if (no_options(o) && (dt == DT_I4 || dt == DT_FP4) && M > small_m && M <= 4096 && (double)M * N <= (double)(1 << 19) &&
      tiles_of(*p, M, N) * p->ks < (p->ks > 1 ? 128 : 256)) {
    Plan q;
    q.kernel = GP_KERNEL_SPLITK;
    q.Kb = Kb;
    // (MXFP4 not on one wave or 64-byte chunks: 76 x 5568 x 15872 44.4 us on
    // 88 unsplit 64 x 128 tiles against 88.2 on the small-M kernel's 64-byte chunks)
    if (choose_split(dt, bits, M, N, Kb, &q, o) == GP_OK && (dt == DT_I4 || (q.waves > 1 && q.kch > 64))) {
      *p = q;
      return GP_OK;
    }
  }
  // Hot-loop schedule: pinned unless asked otherwise (measured per default
  // tile, one process each: the pinned order was as fast or faster)
  if (o && o->scheduler == 2) {
    if (!o->pipeline && !nosched_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe))
      for (const auto& v : kNoSched)
        if (v.dt == dt && v.ms == p->ms && v.tm == p->tm && v.tn == p->tn && v.tkb == p->tkb) { p->pipe = v.pipe; break; }
    if (p->kg != 1 || p->ks != 1 || !nosched_compiled(dt, p->ms, p->tm, p->tn, p->tkb, p->pipe)) return GP_ESHAPE;
    p->sched = 2;
  }
  if (o && o->epilogue) {
    p->epi = o->epilogue;
  } else {
    // CShuffle (coalesced full-row stores) for tile_n >= 128 when its LDS
    // tile fits the share of the 160 KiB LDS each resident workgroup gets
    // (two per CU, or one for tiles whose accumulators fill half the
    // registers); direct stores otherwise
    const int cbytes = p->tm * (p->tn * ob + 16);
    const int wgs_per_cu = tile_wgs_per_cu(p->tm, p->tn, p->kg);
    p->epi = (p->tn >= 128 && cbytes <= 160 * 1024 / wgs_per_cu) ? EPI_CSHUFFLE : EPI_DIRECT;
  }
  p->xcd = (o && o->xcd_swizzle) ? o->xcd_swizzle : 1;
  return GP_OK;
}

void fill_info(int in_dtype, int64_t M, int64_t N, int64_t K, const Plan& p, gemm_plan_info* out) {
  std::memset(out, 0, sizeof(*out));
  const int bits = elem_bits(in_dtype);
  const int dt = kdt(in_dtype);
  const int ms = p.kernel != GP_KERNEL_SPLITK ? p.ms : 16;
  const int kbm = kernel_mfma_kb(dt, ms);
  const int ob = in_dtype == GP_I8 ? 4 : 2;
  const int bias_lds = 0;   // the plain variant; the fused-epilogue one stages tile_n floats of bias more
  out->kernel = p.kernel;
  out->mfma = ms;
  out->pipeline = p.kernel != GP_KERNEL_SPLITK ? (p.pipe ? p.pipe : 1) : 0;
  out->xcd_swizzle = p.kernel != GP_KERNEL_SPLITK ? p.xcd : 2;
  if (p.kernel == GP_KERNEL_WIDE) {
    out->tile_m = out->tile_n = 256;
    out->tile_k = (int)((int64_t)p.tkb * 8 / bits);
    out->epilogue = p.epi;
    out->waves = 8;
    out->threads = 512;
    const int stages = p.pipe * 512 * p.tkb;                 // A and B tiles per stage
    const int cbytes = p.epi == EPI_CSHUFFLE ? 256 * (256 * 2 + 16) : 0;
    out->lds_bytes = (stages > cbytes ? stages : cbytes) + (dt == DT_FP8 ? 512 * 4 : 0) + bias_lds * 256 * 4;
    out->grid = ((M + 255) / 256) * ((N + 255) / 256);
    out->k_tiles = p.Kb / p.tkb;
    out->mfma_per_wave_tile = (int64_t)(p.tkb / kbm) * (128 / ms) * (64 / ms);
  } else if (p.kernel == GP_KERNEL_TILE) {
    out->tile_m = p.tm;
    out->tile_n = p.tn;
    out->tile_k = (int)((int64_t)p.tkb * 8 / bits);
    out->epilogue = p.epi;
    out->waves = tile_waves(p.tm, p.tn) * p.kg;
    out->threads = 64 * out->waves;
    const int tka = p.tkb * (dt == DT_I4 ? 2 : 1);   // A bytes per row of a K tile
    const bool apart = (p.tm * (tka / 16)) % (64 * tile_waves(p.tm, p.tn)) != 0;
    const int stages = p.pipe ? p.pipe : 2;
    int abuf = p.kg * stages * (p.tm * tka + (apart ? 16 : 0));
    if (dt == DT_FP4) {   // staged E8M0 scales: per stage, or a ring of two slots of SG-tile groups
      if (stages == 2 && p.tkb == 128) {
        // two slots of SG-tile groups (SG / 2 lanes per row, 16 spare bytes for
        // lanes past the rows): SG = 8 where the whole LDS still fits the share
        // of a resident workgroup, else 4
        auto slot = [&](int sg) {
          const int th = 64 * tile_waves(p.tm, p.tn);
          return sg * (p.tm + p.tn) * 8 + (((p.tm * sg / 2) % th || (p.tn * sg / 2) % th) ? 16 : 0);
        };
        const int cb = p.epi == EPI_CSHUFFLE ? p.tm * (p.tn * ob + 16) : 0;
        const int share = 160 * 1024 / tile_wgs_per_cu(p.tm, p.tn, p.kg);
        const int st8 = abuf + 2 * slot(8);
        const int sg = (st8 > cb ? st8 : cb) + bias_lds * p.tn * 4 <= share ? 8 : 4;
        abuf += 2 * slot(sg);
      } else {
        abuf += stages * ((p.tm + p.tn) * (p.tkb / 16) + 16);
      }
    }
    int cbytes = p.epi == EPI_CSHUFFLE ? p.tm * (p.tn * ob + 16) : 0;
    if (p.kg > 1 && p.tm * p.tn * 4 > cbytes) cbytes = p.tm * p.tn * 4;   // K-group reduction
    out->lds_bytes = abuf > cbytes ? abuf : cbytes;
    if (dt == DT_FP8 || dt == DT_I4) out->lds_bytes += 256 * ((p.tm + 63) / 64 + p.tn / 64);  // fp32 scales
    out->lds_bytes += bias_lds * p.tn * 4;
    out->grid = ((M + p.tm - 1) / p.tm) * ((N + p.tn - 1) / p.tn);
    out->k_tiles = p.Kb / p.tkb;
    out->mfma_per_wave_tile = (int64_t)(p.tkb / kbm) * (p.tm / ms) * (p.tn / tile_waves(p.tm, p.tn) / ms);
  } else {
    out->tile_m = 16 * p.mb;
    out->tile_n = 16 * p.nb;
    out->tile_k = (int)((int64_t)p.kch * 8 / bits);
    out->epilogue = GP_EPI_DIRECT;
    out->waves = p.waves;
    out->threads = 64 * p.waves;
    out->lds_bytes = p.waves * p.nb * p.mb * 64 * 16;
    out->grid = (N / (16 * p.nb)) * ((M + 16 * p.mb - 1) / (16 * p.mb));
    out->k_tiles = p.Kb / p.waves / p.kch;
    out->mfma_per_wave_tile = (int64_t)(p.kch / kbm) * p.nb * p.mb;
  }
  // MFMAs the launch issues (the algorithmic (M/ms)(N/ms)(K/K_instr) when
  // the tile divides M and N; edge tiles and partial row blocks add to it)
  out->ksplit = p.ks;
  out->scheduler = p.kernel == GP_KERNEL_SPLITK ? 2 : p.sched;   // the small-M kernel has no fences
  if (p.kernel == GP_KERNEL_TILE && p.ks > 1) {
    out->grid *= p.ks;
    out->k_tiles /= p.ks;
  }
  out->workspace_bytes = workspace_bytes(p, M, N);
  out->mfma_total = out->grid * out->waves * (out->k_tiles / (p.kernel == GP_KERNEL_TILE ? p.kg : 1)) *
                    out->mfma_per_wave_tile;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch[64];

// Last HIP status the library saw in this thread and the runtime call that
// returned it (reported by gemm_last_hip_error / gemm_last_hip_call), and the
// gp_status it maps to.
thread_local hipError_t g_last_hip = hipSuccess;
thread_local const char* g_last_call = "";
int hip_status(hipError_t e, const char* call) {
  g_last_hip = e;
  g_last_call = e == hipSuccess ? "" : call;
  return e == hipSuccess ? GP_OK : GP_EHIP;
}
// HIP keeps one "last error" per thread, set by any runtime call, including
// calls the library did not make (the caller's own, or a framework's). It is
// cleared right before each launch, so that the status read right after the
// launch is the launch's own.
void clear_last_error() { (void)hipGetLastError(); }

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return hip_status(hipErrorInvalidDevice, "hipGetDevice (device index past 63)");
  int v = g_arch[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? GP_OK : GP_EARCH;
}

int launch(int in_dtype, const Plan& p, const void* a, const void* b, const void* sa, const void* sb,
           const float* bias, int act, void* c, int64_t M, int64_t N, void* ws, hipStream_t s) {
  const int dt = kdt(in_dtype);
  hipError_t e;
  clear_last_error();
  if (p.kernel == GP_KERNEL_TILE || p.kernel == GP_KERNEL_WIDE) {
    TileArgs t;
    t.a = (const char*)a;
    t.b = (const char*)b;
    t.sa = sa;
    t.sb = sb;
    t.bias = bias;
    t.c = (char*)c;
    t.M = (uint32_t)M;
    t.N = (uint32_t)N;
    t.Kb = (uint32_t)p.Kb;
    t.tiles_m = (uint32_t)((M + p.tm - 1) / p.tm);
    t.tiles_n = (uint32_t)((N + p.tn - 1) / p.tn);
    t.xcd = p.xcd == 1 ? 1u : 0u;
    t.act = act;
    t.ksplit = (uint32_t)p.ks;
    t.cnt = p.ks > 1 ? (uint32_t*)ws : nullptr;
    t.part = p.ks > 1 ? (char*)ws + kCounterBytes : nullptr;
    const bool fused = bias != nullptr || act != GP_ACT_NONE;
    if (p.kernel == GP_KERNEL_WIDE) {
      switch (dt) {
        case DT_I8: e = launch_wide_i8(p.ms, p.tkb, p.pipe, false, t, s); break;
        case DT_FP8: e = launch_wide_fp8(p.ms, p.tkb, p.pipe, fused, t, s); break;
        case DT_BF16: e = launch_wide_bf16(p.ms, p.tkb, p.pipe, fused, t, s); break;
        case DT_F16: e = launch_wide_f16(p.ms, p.tkb, p.pipe, fused, t, s); break;
        default: e = hipErrorInvalidValue; break;
      }
    } else switch (dt) {
      case DT_I8: e = launch_tile_i8(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, false, p.sched == 1, t, s); break;
      case DT_FP8: e = launch_tile_fp8(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, fused, p.sched == 1, t, s); break;
      case DT_BF16: e = launch_tile_bf16(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, fused, p.sched == 1, t, s); break;
      case DT_F16: e = launch_tile_f16(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, fused, p.sched == 1, t, s); break;
      case DT_FP4: e = launch_tile_fp4(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, fused, p.sched == 1, t, s); break;
      case DT_I4: e = launch_tile_i4(p.ms, p.tm, p.tn, p.tkb, p.pipe, p.epi, p.kg, fused, p.sched == 1, t, s); break;
      default: e = hipErrorInvalidValue; break;
    }
  } else {
    SplitArgs t;
    t.a = (const char*)a;
    t.b = (const char*)b;
    t.sa = sa;
    t.sb = sb;
    t.bias = bias;
    t.c = (char*)c;
    t.M = (uint32_t)M;
    t.N = (uint32_t)N;
    t.Kb = (uint32_t)p.Kb;
    t.act = act;
    switch (dt) {
      case DT_I8: e = launch_splitk_i8(p.nb, p.waves, p.kch, p.mb, t, s); break;
      case DT_FP8: e = launch_splitk_fp8(p.nb, p.waves, p.kch, p.mb, t, s); break;
      case DT_BF16: e = launch_splitk_bf16(p.nb, p.waves, p.kch, p.mb, t, s); break;
      case DT_F16: e = launch_splitk_f16(p.nb, p.waves, p.kch, p.mb, t, s); break;
      case DT_I4: e = launch_splitk_i4(p.nb, p.waves, p.kch, p.mb, t, s); break;
      default: e = launch_splitk_fp4(p.nb, p.waves, p.kch, p.mb, t, s); break;
    }
  }
  return hip_status(e, "kernel launch");
}

// B preshuffle: one thread per destination 16-byte chunk (writes coalesced;
// a wave reads 16 rows x 64 contiguous bytes). For INT4 weights the nibbles
// of each 16-byte piece are also reordered: element t of the piece's 32 goes
// to byte t % 16, low nibble for t < 16, high nibble otherwise.
__global__ __launch_bounds__(256) void preshuffle_kernel(const char* __restrict__ b, char* __restrict__ bs,
                                                         uint32_t kb64, uint32_t Kb, uint32_t chunks, int int4) {
  const uint32_t q = blockIdx.x * 256u + threadIdx.x;
  if (q >= chunks) return;
  const uint32_t j = q & 15u;
  const uint32_t g = (q >> 4) & 3u;
  const uint32_t t = q >> 6;
  const uint32_t k0 = t % kb64;
  const uint32_t n0 = t / kb64;
  const size_t src = (size_t)(16u * n0 + j) * Kb + 64u * k0 + 16u * g;
  v4i v = *(const v4i*)(b + src);
  if (int4) {
    // source byte i holds elements 2i (low nibble) and 2i+1 (high nibble)
    v4i o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t w = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int e_lo = 4 * d + bb, e_hi = 16 + 4 * d + bb;   // elements of output byte 4d + bb
        const uint32_t lo = ((uint32_t)v[e_lo >> 3] >> (4 * (e_lo & 7))) & 0xFu;
        const uint32_t hi = ((uint32_t)v[e_hi >> 3] >> (4 * (e_hi & 7))) & 0xFu;
        w |= (lo | (hi << 4)) << (8 * bb);
      }
      o[d] = (int)w;
    }
    v = o;
  }
  *(v4i*)(bs + (size_t)q * 16u) = v;
}

// Every GEMM entry point lands here: validation (pointers, dtype pair,
// scales, epilogue), the plan, the device check, the launch.
// ---- the library's own workspace, for the allocation-free entry point ----
// One static device array (per device: each device that loads the library's
// code holds its own copy until the process ends). Host code never uses its
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
constexpr int64_t kScratchBytes = ((int64_t)32 << 20) + kCounterBytes;
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

// Device address of the current device's scratch array; on the first call
// on a device its counter area is cleared by a fill kernel on `s` (ordered
// before the GEMM that follows on the same stream).
int scratch_for_current_device(void** out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return hip_status(hipErrorInvalidDevice, "hipGetDevice (device index past 63)");
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&] {
    void* ptr = nullptr;
    hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r == hipSuccess) {
      clear_last_error();
      const uint32_t words = (uint32_t)(kCounterBytes / 4);
      hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s, (uint32_t*)ptr, words);
      r = hipGetLastError();
    }
    sl.err = r;
    sl.ptr = r == hipSuccess ? ptr : nullptr;
  });
  if (sl.err != hipSuccess) return hip_status(sl.err, "scratch set-up (hipGetSymbolAddress, fill kernel)");
  *out = sl.ptr;
  return GP_OK;
}

// ws_mode: 0 no workspace (never split), 1 the caller's (ws, ws_bytes),
// 2 the library's static scratch array.
int run_gemm(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
             const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
             const gemm_opts* opts, void* stream, int ws_mode = 0, void* ws = nullptr, size_t ws_bytes = 0) {
  if (!a || !b_shuf || !c || !aligned16(a) || !aligned16(b_shuf) || !aligned16(c)) return GP_EINVAL;
  if (act < GP_ACT_NONE || act > GP_ACT_GELU) return GP_EINVAL;
  if (bias && !aligned16(bias)) return GP_EINVAL;
  bool scales;   // the type takes (required) scale vectors
  switch (in_dtype) {
    case GP_I8:
      // exact int32 result: no scales and no fused epilogue
      if (out_dtype != GP_I32 || bias || act != GP_ACT_NONE) return GP_EDTYPE;
      scales = false;
      break;
    case GP_FP8_E4M3:
    case GP_FP4_E2M1:
    case GP_I4: if (out_dtype != GP_BF16) return GP_EDTYPE; scales = true; break;
    case GP_BF16: if (out_dtype != GP_BF16) return GP_EDTYPE; scales = false; break;
    case GP_F16: if (out_dtype != GP_F16) return GP_EDTYPE; scales = false; break;
    default: return GP_EDTYPE;
  }
  if (scales) {
    if (!scale_a || !scale_b) return GP_EDTYPE;
    if (!aligned16(scale_a) || !aligned16(scale_b)) return GP_EINVAL;
  } else if (scale_a || scale_b) {
    return GP_EDTYPE;
  }
  Plan p;
  int r = make_plan(in_dtype, M, N, K, opts, &p, ws_mode != 0);
  if (r) return r;
  // the scheduler-off variants have the plain epilogue only (the K-split
  // ones have both)
  if (p.sched == 2 && (bias || act != GP_ACT_NONE)) return GP_ESHAPE;
  const int64_t need = workspace_bytes(p, M, N);
  if (need > 0 && ws_mode == 2) {
    if (need > kScratchBytes) return GP_EWORKSPACE;   // more than the static array holds
  } else if (need > 0) {
    if (!ws || (int64_t)ws_bytes < need) return GP_EWORKSPACE;
    if (!aligned16(ws)) return GP_EINVAL;
  }
  r = check_device();
  if (r) return r;
  if (need > 0 && ws_mode == 2) {
    r = scratch_for_current_device(&ws, (hipStream_t)stream);
    if (r) return r;
  }
  return launch(in_dtype, p, a, b_shuf, scale_a, scale_b, bias, act, c, M, N, ws, (hipStream_t)stream);
}

}  // namespace
}  // namespace gp

using namespace gp;

extern "C" {

const char* gemm_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

const char* gemm_last_hip_call(void) { return g_last_call; }

const char* gemm_status_string(int status) {
  switch (status) {
    case GP_OK: return "ok";
    case GP_EINVAL: return "invalid argument (null/misaligned pointer, non-positive size or bad option)";
    case GP_ESHAPE: return "shape not supported (layout or tile divisibility, or size limit)";
    case GP_EDTYPE: return "unsupported dtype or dtype/scale combination";
    case GP_EARCH: return "current device is not gfx950";
    case GP_EHIP: return "HIP runtime or launch error";
    case GP_EWORKSPACE: return "the plan needs a workspace (gemm_ex_ws) of at least gemm_workspace_size bytes";
    default: return "unknown status";
  }
}

int gemm_plan(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, gemm_plan_info* out) {
  if (!out) return GP_EINVAL;
  Plan p;
  const int r = make_plan(in_dtype, M, N, K, opts, &p);
  if (r) return r;
  fill_info(in_dtype, M, N, K, p, out);
  return GP_OK;
}

int gemm_preshuffle_b(const void* b, void* b_shuf, int64_t N, int64_t K, int dtype, void* stream) {
  if (!b || !b_shuf || !aligned16(b) || !aligned16(b_shuf) || N <= 0 || K <= 0) return GP_EINVAL;
  const int bits = elem_bits(dtype);
  if (bits == 0) return GP_EDTYPE;
  if (N >= kMaxBytes || K >= kMaxBytes || (K * bits) % 8) return GP_ESHAPE;
  const int64_t Kb = K * bits / 8;
  if (N % 16 || Kb % 64 || !fits(N, Kb)) return GP_ESHAPE;
  const char* bb = (const char*)b;
  const char* be = bb + N * Kb;
  const char* sb = (const char*)b_shuf;
  if (sb < be && bb < sb + N * Kb) return GP_EINVAL;  // overlap
  const int r = check_device();
  if (r) return r;
  const uint32_t chunks = (uint32_t)(N * Kb / 16);
  clear_last_error();
  hipLaunchKernelGGL(preshuffle_kernel, dim3((chunks + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                     (const char*)b, (char*)b_shuf, (uint32_t)(Kb / 64), (uint32_t)Kb, chunks,
                     dtype == GP_I4 ? 1 : 0);
  return hip_status(hipGetLastError(), "kernel launch");
}

int gemm_a8w8(const void* a, const void* b_shuf, const float* scale_a, const float* scale_b, void* c,
              int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, const gemm_opts* opts,
              void* stream) {
  if (in_dtype != GP_I8 && in_dtype != GP_FP8_E4M3) return GP_EDTYPE;
  return run_gemm(in_dtype, out_dtype, a, b_shuf, scale_a, scale_b, nullptr, GP_ACT_NONE, c, M, N, K, opts, stream);
}

int gemm_bf16(const void* a, const void* b_shuf, void* c, int64_t M, int64_t N, int64_t K,
              const gemm_opts* opts, void* stream) {
  return run_gemm(GP_BF16, GP_BF16, a, b_shuf, nullptr, nullptr, nullptr, GP_ACT_NONE, c, M, N, K, opts, stream);
}

int gemm_mxfp4(const void* a, const uint8_t* scale_a, const void* b_shuf, const uint8_t* scale_b, void* c,
               int64_t M, int64_t N, int64_t K, const gemm_opts* opts, void* stream) {
  if (!scale_a || !scale_b) return GP_EINVAL;
  return run_gemm(GP_FP4_E2M1, GP_BF16, a, b_shuf, scale_a, scale_b, nullptr, GP_ACT_NONE, c, M, N, K, opts,
                  stream);
}

int gemm_f16(const void* a, const void* b_shuf, void* c, int64_t M, int64_t N, int64_t K,
             const gemm_opts* opts, void* stream) {
  return run_gemm(GP_F16, GP_F16, a, b_shuf, nullptr, nullptr, nullptr, GP_ACT_NONE, c, M, N, K, opts, stream);
}

int gemm_w4a8(const void* a, const void* b_shuf, const float* scale_a, const float* scale_b, void* c,
              int64_t M, int64_t N, int64_t K, const gemm_opts* opts, void* stream) {
  return run_gemm(GP_I4, GP_BF16, a, b_shuf, scale_a, scale_b, nullptr, GP_ACT_NONE, c, M, N, K, opts, stream);
}

int gemm_ex(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
            const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
            const gemm_opts* opts, void* stream) {
  return run_gemm(in_dtype, out_dtype, a, b_shuf, scale_a, scale_b, bias, act, c, M, N, K, opts, stream);
}

int gemm_plan_ws(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, gemm_plan_info* out) {
  if (!out) return GP_EINVAL;
  Plan p;
  const int r = make_plan(in_dtype, M, N, K, opts, &p, true);
  if (r) return r;
  fill_info(in_dtype, M, N, K, p, out);
  return GP_OK;
}

int gemm_workspace_size(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, size_t* bytes) {
  if (!bytes) return GP_EINVAL;
  Plan p;
  const int r = make_plan(in_dtype, M, N, K, opts, &p, true);
  if (r) return r;
  *bytes = (size_t)workspace_bytes(p, M, N);
  return GP_OK;
}

int gemm_ex_ws(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
               const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
               const gemm_opts* opts, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gemm(in_dtype, out_dtype, a, b_shuf, scale_a, scale_b, bias, act, c, M, N, K, opts, stream, 1,
                  workspace, workspace_bytes);
}

int gemm_ex_noalloc(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
                    const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
                    const gemm_opts* opts, void* stream) {
  return run_gemm(in_dtype, out_dtype, a, b_shuf, scale_a, scale_b, bias, act, c, M, N, K, opts, stream, 2);
}

}  // extern "C"
