// LDS ping-pong tile kernel for the preshuffle GEMM on gfx950.
//
// Structure (GEMM Optimization Guide §1-§7, Kernel Tuning Guide §1-§6):
//   * one workgroup = 4 waves x 64 lanes computes a TM x TN tile of C; the
//     waves split TN (each owns TN/4 columns) and share the A tile (§1.1);
//     with KG = 2, two such groups split the K tiles and add their results;
//   * A goes global -> VGPR -> LDS into one of two LDS buffers (ping-pong,
//     §2; PIPE = 0), or global -> LDS by the buffer-load LDS DMA into PIPE
//     buffers (async copy, Kernel Tuning Guide §4; PIPE = 2 .. 6), with an
//     XOR swizzle on 16-byte chunks (§3);
//   * B goes global -> VGPR directly from the preshuffled layout (§4.2), in
//     one register set per pipeline stage;
//   * the loads of the tile PIPE-1 ahead are issued during the current
//     tile's MFMAs (loop-carried, §4.1-§4.4); one barrier per K tile;
//   * W4A8: each INT4 B piece is widened in registers to two int8 operands
//     and feeds two int8 MFMAs; the A tile holds two bytes per B byte;
//   * epilogue: direct store or CShuffle through LDS (§7), with the fused
//     bias and activation of Kernel Tuning Guide §6;
//   * M and N need not be multiples of the tile: an edge tile is moved back
//     to end at the last row / column (it overlaps its neighbour) and stores
//     only the rows / columns its neighbour did not, so every load stays
//     inside the operands and the K loop is the same for every tile.
//
// Differences from the pages' kernel, for gfx950:
//   * MS x MS MFMA blocks with MS = 16 or 32 (see Mma<> in gp_common.hpp):
//     the K-doubled gfx950 instructions, and the 32x32 forms (INT8, BF16,
//     FP16, FP4: twice the FLOPs per instruction, fewer operand reads);
//   * the MFMA takes B as its first operand and A as its second, so a lane
//     ends up holding runs of 4 consecutive COLUMNS of one row of C; the
//     direct store is then one 8-byte (bf16) or 16-byte (int32) store;
//   * the swizzle folds (row / P) into the chunk index, P = rows per 256-byte
//     LDS bank period: on 64 banks this makes the 16 rows read by one
//     16-lane phase hit 16 distinct 16-byte bank groups for every row length.
#pragma once

#include <type_traits>

#include "gp_common.hpp"

namespace gp {

struct TileArgs {
  const char* a;      // [M][Kb] (W4A8: [M][2 Kb])
  const char* b;      // preshuffled [N/16][Kb/64][4][16][16]
  const void* sa;     // FP8, W4A8: fp32 [M]; FP4: u8 [M][Kb/16]; else unused
  const void* sb;     // FP8, W4A8: fp32 [N]; FP4: u8 [N][Kb/16]; else unused
  const float* bias;  // fp32 [N] or null (fused epilogue; not INT8)
  char* c;            // [M][N] int32, bf16 or fp16
  uint32_t M, N, Kb;  // Kb = bytes per row of B (and of A, except W4A8: 2 Kb)
  uint32_t tiles_m, tiles_n;  // ceil(M / TM), ceil(N / TN)
  uint32_t xcd;       // 1: XCD-aware, grouped tile order
  int act;            // Act
  // K split across workgroups (tile kernel): ksplit workgroups share each
  // tile, each taking a contiguous range of its K tiles; their partial sums
  // meet in `part` and the last one to finish adds them and stores the tile.
  uint32_t ksplit;    // 1: no split
  char* part;         // [tiles][ksplit][TM*TN] fp32 / int32 partial tiles
  uint32_t* cnt;      // [tiles] arrival counters: zero before, zero after
};

// Edge tiles: a tile that would run past M (or N) starts TM (TN) before the
// end instead; `skip` rows (columns) at its start belong to the previous
// tile and are not stored again.
// Both results are wave-uniform; readfirstlane keeps them in scalar registers
// (left alone, the compiler may pick a vector saturating subtract, and every
// buffer resource built from x0 would then need a waterfall loop).
__device__ __forceinline__ void edge_shift(uint32_t& x0, uint32_t& skip, uint32_t T, uint32_t X) {
  const uint32_t s = x0 + T > X ? x0 + T - X : 0u;
  skip = __builtin_amdgcn_readfirstlane(s);
  x0 = __builtin_amdgcn_readfirstlane(x0 - s);
}

// Resident workgroups per CU of the tile kernel: one once the accumulators
// alone take more than half of the 256 registers two workgroups would leave
// each wave, or with two K groups; two otherwise.
constexpr int tile_wgs_per_cu(int tm, int tn, int kg) { return (kg > 1 || tn >= 512 || tm * tn / 256 > 128) ? 1 : 2; }

// Waves of one K group: 4, each owning TN / 4 columns; 8 for TN = 512, so
// that each wave keeps the 64 columns (and accumulator registers) of the
// 4-wave 256-column tile while one A tile in LDS serves twice the columns:
// a quarter fewer operand bytes from L2 per FLOP than two 128 x 256 tiles.
// 8 also for 256 x 256 tiles: each wave owns 32 columns of all 256 rows
// (the same 128 accumulator registers per lane), so every B byte a wave
// loads feeds 256 rows (half the B bytes per FLOP of the 128 x 512 tile)
// while every wave reads the whole A tile from LDS.
constexpr int tile_waves(int tm, int tn) { return (tn >= 512 || (tm >= 256 && tn >= 256)) ? 8 : 4; }

// PIPE: 0 = A staged through VGPRs, two LDS buffers (prefetch one tile
// ahead); 2 .. 6 = A copied global -> LDS by the buffer-load LDS DMA, with
// PIPE LDS buffers and B register sets (prefetch PIPE-1 tiles ahead).
// FUSED: the variant with the fused bias / activation epilogue; without it
// the epilogue carries no bias slot and no activation code.
// KG: K groups. With KG = 2 the workgroup is two groups of 4 waves that run
// the same tile pipeline on the two halves of the K tiles, each with its own
// LDS stages, and add their accumulators through LDS at the end: twice the
// waves and loads in flight per CU at the same bytes per FLOP, for grids of
// about one tile per CU (THREADS, WAVES and `tid` below are per group).
template <int DT, int MS, int TM, int TN, int TKB, int EPI, int PIPE, bool FUSED = false, int KG = 1>
struct TileCfg {
  using S = Mma<DT, MS>;
  static constexpr int WAVES = tile_waves(TM, TN);
  static constexpr int THREADS = 64 * WAVES;
  // W4A8 (DT_I4): TKB counts bytes of B; A holds two bytes (int8) per B byte
  // (two INT4), and one 16-byte B piece feeds two int8 MFMAs.
  static constexpr int AKB = (DT == DT_I4) ? 2 : 1;        // A bytes per B byte of K
  static constexpr int KB = S::KB;                        // B K bytes per MFMA step
  static constexpr int FRAG = S::FRAG;                    // 16-byte B pieces per lane per step
  static constexpr int AFRAG = (DT == DT_I4) ? 2 : FRAG;  // 16-byte A pieces per lane per step
  static constexpr int TKA = TKB * AKB;                   // A bytes per row of one K tile
  static constexpr int KSTEPS = TKB / KB;
  static constexpr int MREP = TM / MS;
  static constexpr int NPW = TN / WAVES;
  static constexpr int NACC = NPW / MS;
  static constexpr int NREG = S::NREG;
  static constexpr int CPR = TKA / 16;                    // 16-byte chunks per A row
  static constexpr int ACHUNKS = TM * CPR;
  static constexpr int ALOADS = (ACHUNKS + THREADS - 1) / THREADS;
  static constexpr bool APART = (ACHUNKS % THREADS) != 0;
  static constexpr bool ASYNC = PIPE != 0;
  static constexpr int ST = ASYNC ? PIPE : 2;              // pipeline stages
  static constexpr int ABUF = TM * TKA + (APART ? 16 : 0);   // + a spare slot for idle lanes
  static constexpr int OB = (DT == DT_I8) ? 4 : 2;        // output element bytes
  static constexpr bool FSC = DT == DT_FP8 || DT == DT_I4;  // fp32 row / column scales
  static constexpr int CSTRIDE = TN * OB + 16;            // padded C row in LDS
  static constexpr int CBYTES = (EPI == EPI_CSHUFFLE) ? TM * CSTRIDE : 0;
  static constexpr int SWP = (TKA >= 256) ? 1 : 256 / TKA;  // rows per 256-byte period
  static constexpr int SWM = ((CPR < 16) ? CPR : 16) - 1;   // chunk xor mask
  static constexpr int NSC = (DT == DT_FP4) ? 1 : 0;
  // FP4 E8M0 scales of one K tile: one byte per 16 K-bytes (32 elements), so
  // SCB = TKB/16 bytes per row of A and of B, staged in LDS beside the A tile
  // as [row][lane group] entries whose byte s is the scale of K step s:
  //   MS = 16: 4 lane groups x 2 bytes (KSTEPS <= 2); MS = 32: 2 x 4 bytes.
  static constexpr int SCB = NSC ? TKB / 16 : 0;
  static constexpr int SROWS = NSC ? TM + TN : 0;
  // Scale groups: with a 2-stage pipeline and 8 scale bytes per row per tile,
  // the scales of SG consecutive K tiles are fetched together (16 bytes per
  // lane, SG/2 lanes per row) into a two-slot LDS ring. A tile's TM + TN
  // scale rows are as many separate cache lines; one gather of them per tile
  // cost the texture path about as much as the tile's operand loads (the
  // MXFP4 4096x4096x8192 kernel ran 15% faster with the gathers removed).
  // The NGL loads of a thread for group g+1 are spread over the SG tiles of
  // group g, one or two per tile, each staged at the end of its tile (the
  // main loop runs SG tiles per trip, so every tile knows its share at
  // compile time). SG = 8 where both slots fit the LDS share of a resident
  // workgroup, else 4.
  static constexpr bool GROUPED = NSC && ST == 2 && SCB == 8;
  // staged bytes of one tile. Rows are permuted inside each tile of a group:
  // tiles 2p and 2p+1 (written by the group loads of piece p) hold row r at
  // position r ^ 8p. The LPR pieces of one row sit a multiple of 256 bytes
  // apart, so unpermuted every piece of a row hit the same LDS banks (a
  // 4-way conflict on every scale write); permuted, piece p lands 16 p banks
  // further on. The XOR stays inside a 32-row block, and every reader's row
  // base is a multiple of 32.
  static constexpr int GTILE = SROWS * 8;
  static constexpr int LDS_SHARE = 160 * 1024 / tile_wgs_per_cu(TM, TN, KG);
  static constexpr int slot_bytes(int sg) {
    return sg * GTILE + ((((TM * sg / 2) % THREADS) || ((TN * sg / 2) % THREADS)) ? 16 : 0);
  }
  static constexpr int lds_with(int sg) {
    const int stage = KG * ST * ABUF + 2 * slot_bytes(sg);
    const int cb = (EPI == EPI_CSHUFFLE) ? TM * CSTRIDE : 0;
    return (stage > cb ? stage : cb) + ((FUSED && DT != DT_I8) ? TN / 64 * 256 : 0);
  }
  static constexpr int SG = !GROUPED ? 1 : (lds_with(8) <= LDS_SHARE ? 8 : 4);
  static constexpr int LPR = SG > 1 ? SG * SCB / 16 : 0;                     // 16-byte lanes per row
  static constexpr int GLA = SG > 1 ? (TM * LPR + THREADS - 1) / THREADS : 0;  // group loads per thread
  static constexpr int GLB = SG > 1 ? (TN * LPR + THREADS - 1) / THREADS : 0;
  static constexpr int NGL = GLA + GLB;
  // group loads [gl_first(p), gl_first(p+1)) run in the tile at group position p
  static constexpr int gl_first(int p) { return (p * NGL + SG - 1) / (SG > 1 ? SG : 1); }
  static constexpr int GPP = SG > 1 ? (NGL + SG - 1) / SG : 0;               // most per tile
  // a spare 16 bytes after the tiles of a slot for lanes past the last row
  static constexpr bool GSPARE = SG > 1 && (((TM * LPR) % THREADS) || ((TN * LPR) % THREADS));
  static constexpr int GSLOT = SG > 1 ? slot_bytes(SG) : 0;
  static constexpr bool PERTILE = NSC && SG == 1;  // otherwise: scale loads with each tile
  static constexpr int SLA = PERTILE ? (TM + THREADS - 1) / THREADS : 0;   // A scale rows per thread
  static constexpr int SLB = PERTILE ? (TN + THREADS - 1) / THREADS : 0;   // B scale rows per thread
  static constexpr int SLOADS = SLA + SLB;
  static constexpr int SAREA = PERTILE ? SROWS * SCB + 16 : 0;   // + a spare slot for idle lanes
  static constexpr int GSTAGE = ST * ABUF;                            // A stages of one K group
  static constexpr int STAGE = KG * GSTAGE + ST * SAREA + 2 * GSLOT;  // scale ring: 2 slots
  // FP8 / W4A8 per-row / per-column scales, fetched into LDS by DMA when the kernel
  // starts (so the epilogue does not wait a memory round trip for them):
  // 256-byte blocks of A scales (TM floats, padded to 64) then B scales.
  // The fused-epilogue bias (TN floats) follows them.
  static constexpr int NSA = FSC ? (TM + 63) / 64 : 0;
  static constexpr int NSB = FSC ? TN / 64 : 0;
  static constexpr int NBI = (FUSED && DT != DT_I8) ? TN / 64 : 0;
  // K groups: the second group's accumulators, [register chunk][lane] v4 entries
  static constexpr int REDB = KG > 1 ? 256 * (TM * TN / 256) * 4 : 0;
  static constexpr int EPIB = CBYTES > REDB ? CBYTES : REDB;
  static constexpr int FSC_OFF = (STAGE > EPIB) ? STAGE : EPIB;
  static constexpr int BIAS_OFF = FSC_OFF + (NSA + NSB) * 256;
  static constexpr int LDS = BIAS_OFF + NBI * 256;
  // A fragments read ahead of their MFMAs: the most (2, 1 or 0) for which
  // the register estimate (accumulators unless they sit in AGPRs, B stages,
  // FP4 scales, the fragment ring) stays within 236 of the 256 VGPRs. FP8
  // stops at 1: one FP8 fragment feeds NACC 32-cycle MFMAs, which covers an
  // LDS read on its own.
  static constexpr int ACCR = TM * TN / THREADS;
  static constexpr int BREG = ST * KSTEPS * NACC * FRAG * 4 + (DT == DT_I4 ? NACC * 8 : 0);  // + widened INT4
  static constexpr int SREG = NSC ? MREP + NACC + 2 * ST * (SLA + SLB) + 4 * GPP : 0;
  static constexpr int RBASE = (ACCR > 128 ? 0 : ACCR) + BREG + SREG;
  static constexpr int RA = (AFRAG == 1 && RBASE + 12 <= 236) ? 2 : (RBASE + 2 * AFRAG * 4 <= 236) ? 1 : 0;
  static_assert(TM % MS == 0 && NPW % MS == 0 && TN % 64 == 0, "tile shape");
  static_assert(TKB % KB == 0 && TKB >= 64, "tile_k bytes must be a multiple of the MFMA K bytes");
  static_assert(THREADS % CPR == 0, "A row chunks must divide the workgroup");
  static_assert(!NSC || TKB == 128 || (MS == 16 && TKB == 64), "FP4 scale staging: 8 (or 4) bytes per row");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(!ASYNC || (!APART && (TM * CPR) % (THREADS * 1) == 0), "LDS DMA covers whole 1 KiB wave blocks");
  static_assert(PIPE == 0 || (PIPE >= 2 && PIPE <= 6), "pipeline");
  static_assert(KG == 1 || (KG == 2 && !NSC), "K groups: not with FP4's staged scales");
  static_assert(DT != DT_I4 || MS == 16, "W4A8: 16 x 16 blocks");
  static_assert(WAVES == 4 || KG == 1, "8-wave tiles: one K group");
};

// Tile (tm, tn) and K split z of this workgroup. With a K split the ksplit
// workgroups of one tile are consecutive in the logical order, so with the
// XCD-aware order they run on the same XCD and meet in its L2.
__device__ __forceinline__ void tile_coords(const TileArgs& p, uint32_t& tm, uint32_t& tn, uint32_t& z) {
  const uint32_t w = blockIdx.x;
  const uint32_t T = p.tiles_m * p.tiles_n;
  const uint32_t S = p.ksplit;
  const uint32_t G = T * S;
  if (p.xcd && (G % 8u) == 0) {
    // Workgroups go round-robin to the 8 XCDs; give each XCD a contiguous
    // range of tiles, then walk it in groups of 8 M-tiles so that the tiles
    // resident together on one XCD share A rows and B columns in its L2.
    const uint32_t logical = (w % 8u) * (G / 8u) + (w / 8u);
    z = logical % S;
    const uint32_t t = logical / S;
    const uint32_t GROUP = 8u;
    const uint32_t per_group = GROUP * p.tiles_n;
    const uint32_t g = t / per_group;
    const uint32_t first_m = g * GROUP;
    const uint32_t gsz = min(GROUP, p.tiles_m - first_m);
    const uint32_t r = t % per_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
  } else {
    z = w % S;
    const uint32_t t = w / S;
    tm = t / p.tiles_n;
    tn = t % p.tiles_n;
  }
}
__device__ __forceinline__ void tile_coords(const TileArgs& p, uint32_t& tm, uint32_t& tn) {
  uint32_t z;
  tile_coords(p, tm, tn, z);
}

// SCH: the hot-loop schedule pinned by scheduling fences (the pages'
// hot_loop_scheduler, GEMM Optimization Guide §5.3; Kernel Tuning Guide §5
// "enable_scheduler"); false leaves the order of the loop body to the
// compiler (same instructions, no fences between the MFMA groups).
// KS: the variant that can split K across workgroups (p.ksplit > 1); the
// others assume p.ksplit == 1 and carry no code for the cross-workgroup sum.
template <int DT, int MS, int TM, int TN, int TKB, int EPI, int PIPE, bool FUSED, int KG, bool SCH = true,
          bool KS = false>
__global__ __launch_bounds__(64 * tile_waves(TM, TN) * KG, tile_wgs_per_cu(TM, TN, KG)) void gemm_tile_kernel(TileArgs p) {
  using C = TileCfg<DT, MS, TM, TN, TKB, EPI, PIPE, FUSED, KG>;
  using Acc = typename Mma<DT, MS>::Acc;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];

  // K group of this wave and the thread index inside its group; everything
  // below indexes by the group-local thread and wave
  const int grp = KG > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x / C::THREADS) : 0;
  const int tid = KG > 1 ? threadIdx.x % C::THREADS : threadIdx.x;
  char* const glds = lds + grp * C::GSTAGE;   // the group's A stages
  // wave index: uniform across the wave; readfirstlane puts it in a scalar
  // register so that offsets derived from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // lane's row / column inside an MFMA block and its K lane group
  const int lrow = lane & (MS - 1);
  const int lgrp = lane / MS;

  uint32_t tm, tn, kz;
  tile_coords(p, tm, tn, kz);
  uint32_t m0 = tm * TM, n0 = tn * TN, mskip, nskip;
  edge_shift(m0, mskip, TM, p.M);
  edge_shift(n0, nskip, TN, p.N);
  const uint32_t Kb = p.Kb;
  const uint32_t Ka = Kb * C::AKB;   // bytes per row of A
  // K tiles of this workgroup: split kz of ksplit equal ranges; of this group:
  // [kt0, kt0 + KT) (the planner makes ksplit * KG divide the K tiles)
  const int KTS = (int)(Kb / TKB) / (KS ? (int)p.ksplit : 1);
  const int KT = KTS / KG;
  const int kt0 = __builtin_amdgcn_readfirstlane((int)kz * KTS + grp * KT);

  // Buffer resources based at this workgroup's first A row / first B block.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * Ka, TM * Ka);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)(n0 / 16) * 16 * Kb, TN * Kb);

  // ---- per-lane constant offsets ----
  // A global -> LDS: thread tid moves chunk (tid % CPR) of rows tid / CPR + i * RPP.
  constexpr int RPP = C::THREADS / C::CPR;  // A rows per pass of the workgroup
  const int arow0 = tid / C::CPR;
  const int ach = tid % C::CPR;
  const uint32_t a_ld0 = arow0 * Ka + ach * 16;
  // the XOR term of rows arow0 + i*RPP does not depend on i when RPP/SWP is a
  // multiple of the swizzle period; then the LDS write offset is a constant step
  constexpr bool AWR_STEP = ((RPP / C::SWP) % (C::SWM + 1)) == 0;
  uint32_t a_wr[AWR_STEP ? 1 : C::ALOADS];
#pragma unroll
  for (int i = 0; i < (AWR_STEP ? 1 : C::ALOADS); ++i) {
    const int row = arow0 + i * RPP;
    a_wr[i] = row * C::TKA + ((ach ^ ((row / C::SWP) & C::SWM)) * 16);
  }
  auto a_wr_off = [&](int i) GP_INLINE -> uint32_t {
    if constexpr (AWR_STEP) return a_wr[0] + i * RPP * C::TKA;
    else return a_wr[i];
  };
  // Lanes past the last A chunk (partial passes only) load from an offset
  // outside the buffer resource (the hardware returns zeros without a memory
  // access) and write to a spare LDS slot, so the K-tile body has no branch.
  auto a_on = [&](int i) GP_INLINE { return !C::APART || i * C::THREADS + tid < C::ACHUNKS; };
  constexpr uint32_t kOOB = 0x80000000u;
  // LDS DMA of A: instruction i of wave w fills the 1 KiB block i*WAVES + w of
  // the A buffer, lane l landing at byte 16*l of it. So lane l fetches the
  // global chunk that belongs at LDS chunk p = (i*WAVES + w)*64 + l: row p/CPR,
  // physical chunk p%CPR, i.e. logical chunk (p%CPR) ^ swizzle(row). The rows
  // of instruction i are those of instruction 0 plus i*RPD, RPD = 256/CPR.
  // Where RPD rows are a whole number of swizzle periods, one source offset
  // serves every instruction (plus i * RPD rows); otherwise (512-byte A rows:
  // 8 rows per instruction, a 16-row swizzle period) each instruction has its own.
  constexpr int RPD = C::THREADS / C::CPR;
  constexpr bool DMA_STEP = (RPD / C::SWP) % (C::SWM + 1) == 0;
  uint32_t a_dma[DMA_STEP ? 1 : C::ALOADS];
  if constexpr (C::ASYNC) {
    const int pch = wave * 64 + lane;
    const int row = pch / C::CPR;
#pragma unroll
    for (int i = 0; i < (DMA_STEP ? 1 : C::ALOADS); ++i) {
      const int r = row + i * RPD;
      a_dma[i] = r * Ka + (((pch % C::CPR) ^ ((r / C::SWP) & C::SWM)) * 16);
    }
  }
  static_assert(!C::ASYNC || RPD * C::ALOADS == TM, "LDS DMA covers the A tile");
  // A K byte (within one MFMA step) of the lane's 16-byte piece f. W4A8: the
  // B piece of lane group g holds K elements [32g, 32g+32) of the step's 128,
  // its low nibbles the first 16 (first MFMA), its high nibbles the rest.
  auto lane_k = [&](int f) GP_INLINE -> int {
    if constexpr (DT == DT_I4) return 32 * lgrp + 16 * f;
    return MS == 16 ? f * 64 + 16 * lgrp : 16 * lgrp;
  };
  // A LDS -> VGPR: lane reads row mi*MS + lrow, chunk (s*KB + lane_k(f)) / 16.
  // The XOR term depends on the row only through lrow (MS*mi/SWP is a whole
  // number of swizzle periods), so one address per (s, f) serves every mi.
  const int swz = (lrow / C::SWP) & C::SWM;
  uint32_t a_rd[C::KSTEPS][C::AFRAG];
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
    for (int f = 0; f < C::AFRAG; ++f)
      a_rd[s][f] = lrow * C::TKA + ((((s * C::KB * C::AKB + lane_k(f)) / 16) ^ swz) * 16);
  // B: column c = wave*NPW + lrow of the wave's first MFMA block lies in
  // 16-column block c/16, lane j = c%16 of it; the lane's K piece is 16-byte
  // group g of a 64-byte K block: offset blk*16*Kb + k0*1024 + g*256 + j*16.
  const int bcol = wave * C::NPW + lrow;
  const uint32_t b_off0 = (uint32_t)(bcol / 16) * 16u * Kb + (uint32_t)(bcol % 16) * 16u + (uint32_t)lgrp * 256u;
  const uint32_t b_step = (uint32_t)(MS / 16) * 16u * Kb;  // next MFMA column block
  // K-step part of the B offset (uniform): MS = 16: K block s*(KB/64)+f; MS = 32:
  // step s covers K bytes [32s, 32s+32) = block s/2, groups 2*(s%2) + lgrp.
  auto b_koff = [&](int s, int f) GP_INLINE -> uint32_t {
    if constexpr (MS == 16) return (uint32_t)(s * (C::KB / 64) + f) * 1024u;
    else return (uint32_t)s * 512u;
  };

  // FP4 block scales: one E8M0 byte per 32 K elements (= 16 bytes of K).
  const uint32_t srow = Kb / 16;  // scale bytes per row
  __amdgpu_buffer_rsrc_t rsa = make_rsrc(nullptr, 0), rsb = make_rsrc(nullptr, 0);
  if constexpr (DT == DT_FP4) {
    rsa = make_rsrc((const char*)p.sa + (size_t)m0 * srow, TM * srow);
    rsb = make_rsrc((const char*)p.sb + (size_t)n0 * srow, TN * srow);
  }

  // FP8 scales and the bias -> LDS, before any operand load: block i by wave
  // i % WAVES, lane l carrying float l of the block (lanes past TM read zeros).
  if constexpr (C::FSC) {
    const __amdgpu_buffer_rsrc_t rfa = make_rsrc((const float*)p.sa + m0, TM * 4);
    const __amdgpu_buffer_rsrc_t rfb = make_rsrc((const float*)p.sb + n0, TN * 4);
#pragma unroll
    for (int i = 0; i < C::NSA + C::NSB; ++i) {
      if (i % C::WAVES != wave || grp != 0) continue;
      char* dst = lds + C::FSC_OFF + i * 256;
      const bool is_a = i < C::NSA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? rfa : rfb, (__attribute__((address_space(3))) void*)dst, 4,
                                               lane * 4 + (is_a ? i : i - C::NSA) * 256, 0, 0, 0);
    }
  }
  // Without a bias its LDS slot holds zeros, so the epilogue adds it without
  // a branch (written before the first barrier, read after the last).
  if constexpr (C::NBI > 0) {
#pragma unroll
    for (int i = 0; i < C::NBI; ++i) {
      if ((C::NSA + C::NSB + i) % C::WAVES != wave || grp != 0) continue;
      if (p.bias) {
        const __amdgpu_buffer_rsrc_t rbi = make_rsrc(p.bias + n0, TN * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbi, (__attribute__((address_space(3))) void*)(lds + C::BIAS_OFF + i * 256),
                                                 4, lane * 4 + i * 256, 0, 0, 0);
      } else {
        *(float*)(lds + C::BIAS_OFF + i * 256 + lane * 4) = 0.f;
      }
    }
  }

  v4i a_st[C::ASYNC ? 1 : C::ALOADS];
  v4i bfr[C::ST][C::KSTEPS][C::NACC][C::FRAG];
  // FP4 scales of each in-flight tile, by stage (stored to LDS one tile ahead),
  // or of the next scale group
  v2i sa_st[C::ST][C::SLA + (C::SLA == 0)], sb_st[C::ST][C::SLB + (C::SLB == 0)];
  Acc acc[C::MREP][C::NACC];
#pragma unroll
  for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NACC; ++ni) acc[mi][ni] = Acc{};

  auto load_a = [&](int kt, int i) GP_INLINE {
    if constexpr (!C::ASYNC) a_st[i] = buf_load16(ra, a_on(i) ? a_ld0 : kOOB, kt * C::TKA + i * RPP * Ka);
  };
  auto store_a = [&](int par) GP_INLINE {
    if constexpr (C::ASYNC) return;
    char* base = glds + par * C::ABUF;
#pragma unroll
    for (int i = 0; i < C::ALOADS; ++i)
      *(v4i*)(base + (a_on(i) ? a_wr_off(i) : (uint32_t)(TM * C::TKA))) = a_st[i];
  };
  auto load_a_dma = [&](int stage, int kt, int i) GP_INLINE {
    if constexpr (C::ASYNC)
      lds_dma16(p.a + (size_t)m0 * Ka, TM * Ka, glds + stage * C::ABUF + (i * C::WAVES + wave) * 1024,
                (DMA_STEP ? a_dma[0] + i * RPD * Ka : a_dma[DMA_STEP ? 0 : i]) + kt * C::TKA);
  };
  // B load q of a tile: K step q / (NACC*FRAG), column block (q / FRAG) % NACC, piece q % FRAG
  auto load_b = [&](auto par_c, int kt, int q) GP_INLINE {
    constexpr int par = decltype(par_c)::value;
    const int s = q / (C::NACC * C::FRAG), ni = (q / C::FRAG) % C::NACC, f = q % C::FRAG;
    const uint32_t kbase = (uint32_t)kt * (TKB / 64) * 1024u;
    bfr[par][s][ni][f] = buf_load16(rb, b_off0 + b_koff(s, f), kbase + ni * b_step);
  };
  // FP4: the WG's TM + TN scale rows of one K tile, SCB bytes each. A and B
  // rows use separate loads so that each load's buffer resource is uniform.
  // scale load i of a tile: A rows for i < SLA, then B rows
  auto load_s = [&](int st, int kt, int i) GP_INLINE {
    if constexpr (DT == DT_FP4) {
      const uint32_t sbase = (uint32_t)kt * C::SCB;
      if (i < C::SLA) {
        const int r = i * C::THREADS + tid;
        const uint32_t off = r < TM ? r * srow : kOOB;
        if constexpr (C::SCB == 8) sa_st[st][i] = buf_load8(rsa, off, sbase);
        else sa_st[st][i][0] = buf_load4(rsa, off, sbase);
      } else {
        const int r = (i - C::SLA) * C::THREADS + tid;
        const uint32_t off = r < TN ? r * srow : kOOB;
        if constexpr (C::SCB == 8) sb_st[st][i - C::SLA] = buf_load8(rsb, off, sbase);
        else sb_st[st][i - C::SLA][0] = buf_load4(rsb, off, sbase);
      }
    }
  };
  // The 8 scale bytes of one row of one tile (byte b: K bytes [16b, 16b+16))
  // rearranged into [lane group] entries whose byte s is the scale of K step s.
  auto perm_s = [&](v2i v) GP_INLINE -> v2i {
    v2i w;
    if constexpr (MS == 16) {
      // group g (K step s uses block 4s+g): u16 (b_g, b_{4+g})
      w[0] = (int)__builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x05010400u);
      w[1] = (int)__builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x07030602u);
    } else {
      // group q (K step s uses block 2s+q): u32 (b_q, b_{2+q}, b_{4+q}, b_{6+q})
      w[0] = (int)__builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x06040200u);
      w[1] = (int)__builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x07050301u);
    }
    return w;
  };
  // scale row r (A rows first, then B rows) -> LDS as [row][lane group];
  // row SROWS is the spare slot of idle lanes.
  auto put_s = [&](char* base, int r, v2i v) GP_INLINE {
    if constexpr (C::SCB == 8) *(v2i*)(base + r * 8) = perm_s(v);
    else *(int*)(base + r * 4) = v[0];
  };
  // Scale group g (tiles SG*g .. SG*g+SG-1): group load j of a thread (A
  // rows for j < GLA, then B rows; i = its index within them) covers
  // lane-load q = i*THREADS + tid, row q / LPR, 16-byte piece q % LPR, i.e.
  // tiles 2*piece and 2*piece+1 of the group. The whole offset (row and K)
  // is the per-lane one, so that a piece past the end of the scale rows (the
  // last group of a K not a multiple of SG tiles) reads zeros.
  // g < 0: every lane reads outside its resource (zeros, no memory access).
  // Per-lane parts of a group load's global and LDS offsets (row tid / LPR,
  // piece tid % LPR of the load's first row); each load adds a uniform part.
  constexpr int GL_LPR = C::LPR > 0 ? C::LPR : 1;
  constexpr int GL_RSTEP = C::THREADS / GL_LPR;   // rows per load
  const uint32_t g_loff = (tid / GL_LPR) * srow + (tid % GL_LPR) * 16;
  const int g_lds = (tid % GL_LPR) * 2 * C::GTILE + ((tid / GL_LPR) ^ (8 * (tid % GL_LPR))) * 8;
  static_assert(C::SG <= 1 || (GL_RSTEP % 32 == 0 && TM % 32 == 0 && 8 * (GL_LPR - 1) < 32),
                "scale row permutation stays inside 32-row blocks");
  auto load_g1 = [&](auto j_c, int g) GP_INLINE -> v4i {
    constexpr int j = decltype(j_c)::value;
    constexpr bool is_a = j < C::GLA;
    constexpr int i = is_a ? j : j - C::GLA;
    bool on = g >= 0;
    if constexpr (C::GSPARE) on = on && i * C::THREADS + tid < (is_a ? TM : TN) * C::LPR;
    const uint32_t u =
        __builtin_amdgcn_readfirstlane(i * GL_RSTEP * srow + (uint32_t)kt0 * C::SCB + (uint32_t)g * (C::SG * C::SCB));
    return buf_load16(is_a ? rsa : rsb, on ? g_loff + u : kOOB, 0);
  };
  // ... into slot `slot` (0 or 1) of the ring: [tile of the group][row][lane group]
  auto store_g1 = [&](auto j_c, int slot, v4i v) GP_INLINE {
    constexpr int j = decltype(j_c)::value;
    constexpr bool is_a = j < C::GLA;
    constexpr int i = is_a ? j : j - C::GLA;
    char* base = lds + C::ST * C::ABUF + slot * C::GSLOT;
    char* d0 = base + g_lds + ((is_a ? 0 : TM) + i * GL_RSTEP) * 8;
    if constexpr (C::GSPARE) {
      if (!(i * C::THREADS + tid < (is_a ? TM : TN) * C::LPR)) d0 = base + C::SG * C::GTILE;   // spare slot
    }
    char* d1 = d0 + ((!C::GSPARE || i * C::THREADS + tid < (is_a ? TM : TN) * C::LPR) ? C::GTILE : 0);
    *(v2i*)d0 = perm_s(v2i{v[0], v[1]});
    *(v2i*)d1 = perm_s(v2i{v[2], v[3]});
  };
  auto store_s = [&](int par) GP_INLINE {
    if constexpr (DT == DT_FP4) {
      char* base = lds + C::ST * C::ABUF + par * C::SAREA;
#pragma unroll
      for (int i = 0; i < C::SLA; ++i) {
        const int r = i * C::THREADS + tid;
        put_s(base, r < TM ? r : C::SROWS, sa_st[par][i]);
      }
#pragma unroll
      for (int i = 0; i < C::SLB; ++i) {
        const int r = i * C::THREADS + tid;
        put_s(base, r < TN ? TM + r : C::SROWS, sb_st[par][i]);
      }
    }
  };
  // lane's scale entry of staged row r
  auto read_s = [&](const char* sbase, int r) GP_INLINE -> int {
    if constexpr (C::SCB == 8) {
      if constexpr (MS == 16) return *(const uint16_t*)(sbase + r * 8 + lgrp * 2);
      else return *(const int*)(sbase + r * 8 + lgrp * 4);
    } else {
      return *(const uint8_t*)(sbase + r * 4 + lgrp);
    }
  };
  // ds_read of A fragment (s, mi) from buffer par
  auto read_a = [&](int par, int s, int mi, v4i* af) GP_INLINE {
    const char* base = glds + par * C::ABUF;
#pragma unroll
    for (int f = 0; f < C::AFRAG; ++f) af[f] = *(const v4i*)(base + a_rd[s][f] + mi * MS * C::TKA);
  };
  // Hot-loop order of one K tile: the first RA A-fragment reads, then for
  // every A fragment i: in the first half of the tile an even share of the
  // global loads of the tile PIPE-1 ahead (scales, A, B), the read of
  // fragment i+RA, fragment i's NACC MFMAs. The A
  // fragments live in a ring of RA+1 register sets, so each ds_read has RA
  // groups of MFMAs to land in. Scheduling fences pin this order: left free,
  // the compiler folds the ring into one register set and waits for every
  // read right before its MFMAs.
  auto fence = [] {
    if constexpr (SCH) __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int NBL = C::KSTEPS * C::NACC * C::FRAG;       // B loads per tile
  constexpr int NVMEM = C::ALOADS + NBL + C::SLOADS;        // global loads per tile
  auto compute = [&](auto par_c, int kt, auto&& issue_loads) GP_INLINE {
    constexpr int par = decltype(par_c)::value;
    // E8M0 scales from LDS: byte s of the value is the scale of K step s
    int psa[C::MREP * C::NSC + 1 - C::NSC], psb[C::NACC * C::NSC + 1 - C::NSC];
    if constexpr (DT == DT_FP4) {
      const char* sb = C::SG > 1 ? lds + C::ST * C::ABUF + ((kt / C::SG) & 1) * C::GSLOT + (kt % C::SG) * C::GTILE
                                 : lds + C::ST * C::ABUF + par * C::SAREA;
      // row r of a grouped tile sits at r ^ xp (bits 3-4 only: the same
      // 32-row block)
      const int xp = C::SG > 1 ? 8 * ((kt % C::SG) / 2) : 0;
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi) psa[mi] = read_s(sb, (mi * MS + lrow) ^ xp);
#pragma unroll
      for (int ni = 0; ni < C::NACC; ++ni) psb[ni] = read_s(sb, (TM + wave * C::NPW + ni * MS + lrow) ^ xp);
    }
    constexpr int NF = C::KSTEPS * C::MREP;
    constexpr int RA = C::RA < NF ? C::RA : NF;
    constexpr int LH = NF > 1 ? NF / 2 : 1;  // groups that carry global loads
    v4i af[RA + 1][C::AFRAG];
    // W4A8: the step's B pieces widened to int8 (once per step, at its first A fragment)
    v4i blo[C::NACC * (DT == DT_I4) + (DT != DT_I4)], bhi[C::NACC * (DT == DT_I4) + (DT != DT_I4)];
#pragma unroll
    for (int j = 0; j < RA; ++j) read_a(par, j / C::MREP, j % C::MREP, af[j]);
    fence();
    static_for<0, NF>([&](auto i_c) GP_INLINE {
      constexpr int i = decltype(i_c)::value;
      constexpr int s = i / C::MREP, mi = i % C::MREP;
      // this group's share of the tile's global loads
      if constexpr (i < LH) issue_loads(std::integral_constant<int, i * NVMEM / LH>{}, std::integral_constant<int, (i + 1) * NVMEM / LH>{});
      if constexpr (i + RA < NF) read_a(par, (i + RA) / C::MREP, (i + RA) % C::MREP, af[(i + RA) % (RA + 1)]);
      fence();
      const v4i* a = af[i % (RA + 1)];
      if constexpr (DT == DT_I4 && mi == 0) {
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni) widen_int4(bfr[par][s][ni][0], blo[ni], bhi[ni]);
      }
#pragma unroll
      for (int ni = 0; ni < C::NACC; ++ni) {
        if constexpr (DT == DT_FP4) {
          acc[mi][ni] = mma<DT, MS, s>(bfr[par][s][ni], a, acc[mi][ni], psb[ni], psa[mi]);
        } else if constexpr (DT == DT_I4) {
          // the widened values are 16 x the INT4 ones; the epilogue divides by 16
          acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(blo[ni], a[0], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bhi[ni], a[1], acc[mi][ni], 0, 0, 0);
        } else {
          acc[mi][ni] = mma<DT, MS>(bfr[par][s][ni], a, acc[mi][ni]);
        }
      }
      fence();
    });
  };
  // s_waitcnt vmcnt(n) alone (expcnt / lgkmcnt left alone)
  auto wait_vm = [&](auto n_c) GP_INLINE {
    constexpr int n = decltype(n_c)::value;
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  // global loads [J0, J1) of one tile, in the fixed order scales, A, B (the
  // wait for A at the end of an iteration counts on that order)
  auto loads = [&](auto stage_c, int kt_in, auto j0_c, auto j1_c) GP_INLINE {
    constexpr int st = decltype(stage_c)::value;
    // the tile index (made global: the group's first tile + the local one) is
    // wave-uniform; say so, so that every offset built from it stays in
    // scalar registers (a VGPR offset would need a waterfall loop)
    const int kt = __builtin_amdgcn_readfirstlane(kt0 + kt_in);
    static_for<decltype(j0_c)::value, decltype(j1_c)::value>([&](auto j_c) GP_INLINE {
      constexpr int j = decltype(j_c)::value;
      if constexpr (j < C::SLOADS) {
        load_s(st, kt, j);
      } else if constexpr (j < C::SLOADS + C::ALOADS) {
        if constexpr (C::ASYNC) load_a_dma(st, kt, j - C::SLOADS);
        else load_a(kt, j - C::SLOADS);
      } else {
        load_b(stage_c, kt, j - C::SLOADS - C::ALOADS);
      }
    });
  };
  using J0 = std::integral_constant<int, 0>;
  using JALL = std::integral_constant<int, NVMEM>;
  // r: stage of tile kt (kt % ST); gpos: kt % SG
  auto iter = [&](auto r_c, auto gpos_c, int kt) GP_INLINE {
    constexpr int r = decltype(r_c)::value;
    constexpr int gpos = decltype(gpos_c)::value;
    constexpr int rn = (r + C::ST - 1) % C::ST;  // stage of the tile ST-1 ahead
    // past the end the last tile reloads itself into a free stage instead of
    // branching, keeping the body one straight-line block
    const int kn = min(kt + C::ST - 1, KT - 1);
    // FP4: this tile's share of the loads of the next scale group, staged at
    // the end of the tile into the slot the previous group left (its last
    // reader, tile SG*(kt/SG)-1, is behind the barrier that ended it). They
    // are issued before the tile's own loads, so the wait at the end of the
    // tile covers them. A group past the last tile reads zeros.
    constexpr int gj0 = C::gl_first(gpos), gj1 = C::gl_first(gpos + 1);
    v4i gv[gj1 > gj0 ? gj1 - gj0 : 1];
    const int gnext = kt / C::SG + 1;
    if constexpr (gj1 > gj0) {
      const int g = gnext * C::SG < KT ? gnext : -1;
      static_for<gj0, gj1>([&](auto j_c) GP_INLINE { gv[decltype(j_c)::value - gj0] = load_g1(j_c, g); });
    }
    compute(r_c, kt, [&](auto j0_c, auto j1_c) GP_INLINE { loads(std::integral_constant<int, rn>{}, kn, j0_c, j1_c); });
    store_a(rn);
    // FP4 scales of the next tile, loaded ST-2 iterations ago (its stage is
    // free: its last reader was tile kt+1-ST)
    store_s((r + 1) % C::ST);
    if constexpr (gj1 > gj0)
      static_for<gj0, gj1>([&](auto j_c) GP_INLINE { store_g1(j_c, gnext & 1, gv[decltype(j_c)::value - gj0]); });
    if constexpr (C::ASYNC) {
      // tile kt+1's DMA was issued ST-2 iterations ago, before that
      // iteration's B loads: everything issued after it may stay in flight
      __builtin_amdgcn_sched_barrier(0);
      wait_vm(std::integral_constant<int, NBL + (C::ST - 2) * NVMEM>{});
    }
    __syncthreads();
  };

  // ---- prologue: tiles 0 .. ST-2 into stages 0 .. ST-2 ----
  v4i g0[C::NGL > 0 ? C::NGL : 1];   // scale group 0
  if constexpr (C::SG > 1) static_for<0, C::NGL>([&](auto j_c) GP_INLINE { g0[decltype(j_c)::value] = load_g1(j_c, 0); });
  static_for<0, C::ST - 1>([&](auto j_c) GP_INLINE {
    constexpr int j = decltype(j_c)::value;
    loads(j_c, min(j, KT - 1), J0{}, JALL{});
    store_a(j);
  });
  store_s(0);
  if constexpr (C::SG > 1) static_for<0, C::NGL>([&](auto j_c) GP_INLINE { store_g1(j_c, 0, g0[decltype(j_c)::value]); });
  if constexpr (C::ASYNC) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm(std::integral_constant<int, NBL + (C::ST - 2) * NVMEM>{});
  }
  __syncthreads();

  // ---- main loop, TRIP K tiles per trip (whole pipeline rounds and scale
  // groups, so that stage and group position are compile-time); the tail
  // has fewer than TRIP tiles and so no group boundary ----
  constexpr int TRIP = C::SG > C::ST ? C::SG : C::ST;
  static_assert(TRIP % C::ST == 0 && TRIP % C::SG == 0, "trip covers whole stages and groups");
  int kt = 0;
  for (; kt + TRIP <= KT; kt += TRIP)
    static_for<0, TRIP>([&](auto r_c) GP_INLINE {
      constexpr int r = decltype(r_c)::value;
      iter(std::integral_constant<int, r % C::ST>{}, std::integral_constant<int, r % C::SG>{}, kt + r);
    });
  static_for<0, TRIP - 1>([&](auto r_c) GP_INLINE {
    constexpr int r = decltype(r_c)::value;
    if (kt + r < KT) iter(std::integral_constant<int, r % C::ST>{}, std::integral_constant<int, r % C::SG>{}, kt + r);
  });
  // no DMA may still be writing LDS when the epilogue reuses it
  if constexpr (C::ASYNC) {
    wait_vm(std::integral_constant<int, 0>{});
    __syncthreads();
  }

  // ---- K groups: the second group's accumulators are added into the first's
  // through LDS (the stages are dead: every DMA has landed and every wave
  // passed the barrier above), in a fixed order ----
  if constexpr (KG > 1) {
    constexpr int NCH = C::MREP * C::NACC * (C::NREG / 4);   // 4-register chunks per lane
    using V4 = std::conditional_t<DT == DT_I8 || DT == DT_I4, v4i, v4f>;
    V4* red = (V4*)lds;
    if (grp == 1) {
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            V4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * h + r];
            red[((mi * C::NACC + ni) * (C::NREG / 4) + h) * 256 + tid] = v;
          }
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            const V4 v = red[((mi * C::NACC + ni) * (C::NREG / 4) + h) * 256 + tid];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][ni][4 * h + r] += v[r];
          }
    }
    static_assert(NCH * 256 * 16 <= C::REDB, "K-group reduction buffer");
    __syncthreads();
  }

  // ---- K split across workgroups: every workgroup of the tile stores its
  // partial sums; the last to arrive adds all of them in the fixed order
  // z = 0 .. ksplit-1, whatever the order of arrival, resets the counter for
  // the next call and runs the epilogue; the others are done. No workgroup
  // waits for another. The partial sums are stored and loaded with the
  // agent-coherent cache policy, each thread's stores are complete before
  // the arrival is counted (a relaxed agent-scope atomic), and the last
  // workgroup loads them only after reading the count: so no cache-wide
  // write-back or invalidate (what a __threadfence costs) is needed. ----
  if constexpr (KS) {
    constexpr int NCH = C::MREP * C::NACC * (C::NREG / 4);   // 4-register chunks per lane
    using V4 = std::conditional_t<DT == DT_I8 || DT == DT_I4, v4i, v4f>;
    const uint32_t tile = tm * p.tiles_n + tn;
    // the tile's partial sums: [z][chunk][thread] 16-byte entries
    constexpr uint32_t PB = NCH * C::THREADS * 16u;   // bytes of one partial tile (TM * TN * 4)
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part + (size_t)tile * p.ksplit * PB, p.ksplit * PB);
    if (grp == 0) {
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            V4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * h + r];
            const uint32_t ch = (mi * C::NACC + ni) * (C::NREG / 4) + h;
            buf_store16_coh(__builtin_bit_cast(v4i, v), rp, ((kz * NCH + ch) * C::THREADS + tid) * 16u);
          }
    }
    wait_vm(std::integral_constant<int, 0>{});   // this thread's partial sums are stored
    __syncthreads();
    volatile uint32_t* arrived = (volatile uint32_t*)lds;
    if (threadIdx.x == 0)
      *arrived = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t before = __builtin_amdgcn_readfirstlane(*arrived);
    __syncthreads();   // every thread has read it before the epilogue reuses the LDS
    if (before != p.ksplit - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (grp == 0) {
      // in batches of RB chunks: the RB loads of one K range are in flight
      // together (one memory round trip per range and batch, not per chunk)
      constexpr int RB = NCH < 8 ? NCH : 8;
      static_assert(NCH % RB == 0, "whole batches of chunks");
      auto get = [&](int ch) GP_INLINE -> V4 {
        const int mi = ch / (C::NACC * (C::NREG / 4)), ni = (ch / (C::NREG / 4)) % C::NACC, h = ch % (C::NREG / 4);
        V4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * h + r];
        return v;
      };
      auto put = [&](int ch, V4 v) GP_INLINE {
        const int mi = ch / (C::NACC * (C::NREG / 4)), ni = (ch / (C::NREG / 4)) % C::NACC, h = ch % (C::NREG / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][4 * h + r] = v[r];
      };
      static_for<0, NCH / RB>([&](auto b_c) GP_INLINE {
        constexpr int c0 = decltype(b_c)::value * RB;
        V4 t[RB], u[RB];
        // partial sums of range z, chunks c0 .. c0+RB-1 (this workgroup's own from registers)
        auto fetch = [&](uint32_t z, V4* dst) GP_INLINE {
          if (z == kz) {
#pragma unroll
            for (int b = 0; b < RB; ++b) dst[b] = get(c0 + b);
          } else {
#pragma unroll
            for (int b = 0; b < RB; ++b)
              dst[b] = __builtin_bit_cast(V4, buf_load16_coh(rp, ((z * NCH + c0 + b) * C::THREADS + tid) * 16u));
          }
        };
        fetch(0, t);
        for (uint32_t zz = 1; zz < p.ksplit; ++zz) {
          fetch(zz, u);
#pragma unroll
          for (int b = 0; b < RB; ++b) t[b] += u[b];
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) put(c0 + b, t[b]);
      });
    }
  }

  // ---- epilogue ---- (the first K group's waves store; a second group only
  // takes part in the barriers)
  // Lane indices re-derived from an opaque copy of the thread index, so that
  // no epilogue address is computed before (and kept live through) the K loop.
  const int etid = opaque(tid);
  const int elrow = etid & (MS - 1), elgrp = (etid & 63) / MS;
  // For every (mi, ni) the lane holds NREG/4 runs of 4 consecutive columns
  // of row mi*MS + elrow: run h covers columns ni*MS + col_run(h) + 0..3.
  auto col_run = [&](int h) GP_INLINE -> int { return MS == 16 ? 4 * elgrp : 8 * h + 4 * elgrp; };
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c + ((size_t)m0 * p.N + n0) * C::OB, ((TM - 1) * p.N + TN) * C::OB);
  // C offset of tile row r, column c; rows / columns an edge tile shares with
  // its neighbour get an offset outside the resource (the store is dropped)
  auto c_off = [&](uint32_t r, uint32_t c) GP_INLINE -> uint32_t {
    return (r >= mskip && c >= nskip) ? (r * p.N + c) * C::OB : 0x80000000u;
  };
  // The scale and bias DMAs were each wave's first memory instructions, so
  // they completed before the wave's wait for any later load (vmcnt counts in
  // order): with DMA A the wait for zero above, with A through VGPRs the wait
  // for the last tile's A. Every wave passed a barrier after that wait.
  v4f sbv[C::NACC][C::NREG / 4];
  float sav[C::MREP];
  if constexpr (C::FSC) {
    const float* sa = (const float*)(lds + C::FSC_OFF);
    const float* sb = sa + C::NSA * 64;
#pragma unroll
    for (int mi = 0; mi < C::MREP; ++mi) sav[mi] = sa[mi * MS + elrow];
#pragma unroll
    for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
      for (int h = 0; h < C::NREG / 4; ++h)
        sbv[ni][h] = *(const v4f*)(sb + wave * C::NPW + ni * MS + col_run(h));
  }
  // bias of a run of 4 columns (read from LDS where it is used)
  auto bias4 = [&](int ni, int h) GP_INLINE -> v4f {
    if constexpr (C::NBI > 0) return *(const v4f*)(lds + C::BIAS_OFF + (wave * C::NPW + ni * MS + col_run(h)) * 4);
    else return v4f{0.f, 0.f, 0.f, 0.f};
  };
  auto out_vec = [&](auto act_c, int mi, int ni, int h, auto emit) GP_INLINE {
    constexpr int A = decltype(act_c)::value;
    if constexpr (DT == DT_I8) {
      v4i v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * h + r];
      emit(v);
    } else {
      v4f v;
      const v4f bv = bias4(ni, h);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x;
        if constexpr (DT == DT_I4) x = (float)(acc[mi][ni][4 * h + r] >> 4);   // exact: a multiple of 16
        else x = acc[mi][ni][4 * h + r];
        if constexpr (C::FSC) x = (x * sav[mi]) * sbv[ni][h][r];
        v[r] = activate<A>(x + bv[r]);
      }
      emit(pack_out4<DT>(v));
    }
  };

  const bool storer = grp == 0;
  auto store_tile = [&](auto act_c) GP_INLINE {
    if constexpr (EPI == EPI_DIRECT) {
      if (!storer) return;
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            const uint32_t off = c_off(mi * MS + elrow, wave * C::NPW + ni * MS + col_run(h));
            out_vec(act_c, mi, ni, h, [&](auto v) GP_INLINE {
              if constexpr (sizeof(v) == 16) buf_store16(v, rc, off);
              else buf_store8(v, rc, off);
            });
          }
    } else {
      // CShuffle: stage the tile in LDS (the A buffers are dead after the last
      // barrier), then write whole rows with 16-byte stores.
      if (storer)
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            char* dst = lds + (mi * MS + elrow) * C::CSTRIDE + (wave * C::NPW + ni * MS + col_run(h)) * C::OB;
            out_vec(act_c, mi, ni, h, [&](auto v) GP_INLINE { *(decltype(v)*)dst = v; });
          }
      __syncthreads();
      constexpr int CH_ROW = TN * C::OB / 16;
      constexpr int TOTAL = TM * CH_ROW;
#pragma unroll
      for (int i = 0; i < (TOTAL + C::THREADS - 1) / C::THREADS; ++i) {
        const int q = i * C::THREADS + etid;
        if ((TOTAL % C::THREADS != 0 && q >= TOTAL) || !storer) break;
        const int row = q / CH_ROW;
        const int ch = q % CH_ROW;
        const v4i v = *(const v4i*)(lds + row * C::CSTRIDE + ch * 16);
        // a 16-byte chunk lies inside one 16-column block: stored whole or not at all
        buf_store16(v, rc, c_off(row, ch * 16 / C::OB));
      }
    }
  };
  if constexpr (FUSED) with_act(p.act, store_tile);
  else store_tile(std::integral_constant<int, ACT_NONE>{});
}

}  // namespace gp
