// Large-tile kernel for the compute-bound shapes on gfx950.
//
// One workgroup of 8 waves per CU computes a 256 x 256 tile of C. The waves
// form a 2 x 4 grid: wave (wm, wn) owns rows [128 wm, 128 wm + 128) and
// columns [64 wn, 64 wn + 64) of the tile. Both operands are copied
// global -> LDS by the buffer-load LDS DMA into PIPE stage buffers, PIPE-1
// K tiles ahead of the MFMAs:
//   * A with the XOR swizzle on 16-byte chunks of the 4-wave tile kernel
//     (GEMM Optimization Guide §3);
//   * B in its preshuffled layout (§1.4): one KiB per 16 columns x 64 K-bytes,
//     so a wave's B fragment is one contiguous KiB of LDS.
// The pages' kernel loads B straight into registers, one copy per wave
// (§4.2). Here the two waves of a column share each B byte through LDS, and
// one CU holds a 256 x 256 tile instead of two 128 x 256 ones: per FLOP a CU
// pulls a third fewer bytes from L2, the path that bounds the 4-wave kernel
// on the large shapes.
//
// Per K tile: for every A fragment i of the wave, in the first half of the
// tile a share of the next tile's DMAs, the read of A fragment i+RA (a ring of
// RA+1 register sets) and, at the start of each MFMA K step, of the next
// step's B fragments, then fragment i's NACC MFMAs; one explicit vmcnt wait
// and one barrier close the tile. Epilogue: FP8 scales and the fused bias
// (DMA'd into LDS at the start), activation, bf16 / fp16 rounding, CShuffle
// through LDS and full-row stores; INT8 stores its int32 results directly.
// Edge tiles of M or N not divisible by 256 are moved back to end at the last
// row / column and store only what their neighbour does not (edge_shift).
#pragma once

#include <type_traits>

#include "gemm_tile.hpp"

namespace gp {

template <int DT, int MS, int TKB, int PIPE, bool FUSED = false>
struct WideCfg {
  using S = Mma<DT, MS>;
  static constexpr int TM = 256, TN = 256;
  static constexpr int WM = 2, WN = 4, WAVES = WM * WN, THREADS = WAVES * 64;
  static constexpr int WTM = TM / WM, WTN = TN / WN;   // 128 x 64 per wave
  static constexpr int KB = S::KB, FRAG = S::FRAG, NREG = S::NREG;
  static constexpr int KSTEPS = TKB / KB;
  static constexpr int MREP = WTM / MS, NACC = WTN / MS;
  static constexpr int KBLK = TKB / 64;                // 64-byte K blocks per tile
  static constexpr int CPR = TKB / 16;                 // 16-byte chunks per A row
  static constexpr int ABYTES = TM * TKB, BBYTES = TN * TKB, STAGE = ABYTES + BBYTES;
  static constexpr int ST = PIPE;
  static constexpr int ADMA = ABYTES / (THREADS * 16);  // DMA instructions per wave per tile
  static constexpr int BDMA = BBYTES / (THREADS * 16);
  static constexpr int NVMEM = ADMA + BDMA;
  static constexpr int RPD = THREADS / CPR;             // A rows per DMA pass
  static constexpr int SWP = (TKB >= 256) ? 1 : 256 / TKB;
  static constexpr int SWM = ((CPR < 16) ? CPR : 16) - 1;
  static constexpr int OB = (DT == DT_I8) ? 4 : 2;
  static constexpr bool CSHUF = DT != DT_I8;            // an int32 C tile does not fit LDS
  static constexpr int CSTRIDE = TN * OB + 16;
  static constexpr int CBYTES = CSHUF ? TM * CSTRIDE : 0;
  static constexpr int PBYTES = ST * STAGE;
  static constexpr int FSC_OFF = PBYTES > CBYTES ? PBYTES : CBYTES;
  static constexpr int BIAS_OFF = FSC_OFF + (DT == DT_FP8 ? (TM + TN) * 4 : 0);
  static constexpr bool BIAS = FUSED && DT != DT_I8;   // bias slot of the fused epilogue
  static constexpr int LDS = BIAS_OFF + (BIAS ? TN * 4 : 0);
  // A fragments read ahead; one FP8 fragment feeds NACC 32-cycle MFMAs,
  // which covers an LDS read on its own
  static constexpr int RA = FRAG == 2 ? 1 : 2;
  static_assert(DT != DT_FP4, "FP4 runs on the 4-wave kernel");
  static_assert(TKB % 64 == 0 && TKB % KB == 0, "whole 64-byte K blocks and MFMA steps");
  static_assert(ADMA * THREADS * 16 == ABYTES && BDMA * THREADS * 16 == BBYTES, "whole DMA passes");
  static_assert((RPD / SWP) % (SWM + 1) == 0, "DMA swizzle step");
  static_assert(PIPE >= 2 && PIPE <= 4, "pipeline");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int DT, int MS, int TKB, int PIPE, bool FUSED>
__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(TileArgs p) {
  using C = WideCfg<DT, MS, TKB, PIPE, FUSED>;
  using Acc = typename Mma<DT, MS>::Acc;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lane = tid & 63;
  const int lrow = lane & (MS - 1);
  const int lgrp = lane / MS;

  uint32_t tm, tn;
  tile_coords(p, tm, tn);
  uint32_t m0 = tm * C::TM, n0 = tn * C::TN, mskip, nskip;
  edge_shift(m0, mskip, C::TM, p.M);
  edge_shift(n0, nskip, C::TN, p.N);
  const uint32_t Kb = p.Kb;
  const int KT = (int)(Kb / TKB);
  const char* ga = p.a + (size_t)m0 * Kb;   // the workgroup's 256 A rows
  const char* gb = p.b + (size_t)n0 * Kb;   // its 16 B column blocks (16 * Kb bytes each)

  // ---- DMA offsets ----
  // A: instruction i of wave w fills KiB block i*WAVES + w of the stage's A
  // tile; lane l lands at byte 16 l, i.e. LDS chunk q = (i*WAVES + w)*64 + l =
  // row q / CPR, physical chunk q % CPR, which holds logical chunk
  // (q % CPR) ^ swizzle(row). Instruction i covers the rows of instruction 0
  // plus i * RPD, a whole number of swizzle periods.
  uint32_t a_dma0;
  {
    const int q = wave * 64 + lane;
    const int row = q / C::CPR;
    a_dma0 = row * Kb + (((q % C::CPR) ^ ((row / C::SWP) & C::SWM)) * 16);
  }
  // B: instruction i of wave w copies KiB block q = i*WAVES + w of the stage's
  // B tile, column block q / KBLK, K block q % KBLK; LDS keeps the global
  // block order, so lane l's 16 bytes go to byte 16 l of block q.
  auto b_dma = [&](int i, int kt) -> uint32_t {
    const int q = i * C::WAVES + wave;
    return (uint32_t)(q / C::KBLK) * 16u * Kb + (uint32_t)(q % C::KBLK + kt * C::KBLK) * 1024u + lane * 16;
  };
  auto dma = [&](int st, int kt, int j) {
    char* stage = lds + st * C::STAGE;
    if (j < C::ADMA)
      lds_dma16(ga, C::TM * Kb, stage + (j * C::WAVES + wave) * 1024, a_dma0 + kt * TKB + j * C::RPD * Kb);
    else
      lds_dma16(gb, C::TN * Kb, stage + C::ABYTES + ((j - C::ADMA) * C::WAVES + wave) * 1024, b_dma(j - C::ADMA, kt));
  };

  // ---- fragment read offsets ----
  // A: lane reads row wm*WTM + mi*MS + lrow, 16-byte chunk (s*KB + lane_k(f)) / 16.
  // wm*WTM + mi*MS is a whole number of swizzle periods, so the XOR term
  // depends on lrow only.
  auto lane_k = [&](int f) -> int { return MS == 16 ? f * 64 + 16 * lgrp : 16 * lgrp; };
  const int swz = (lrow / C::SWP) & C::SWM;
  uint32_t a_rd[C::KSTEPS][C::FRAG];
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
    for (int f = 0; f < C::FRAG; ++f)
      a_rd[s][f] = (wm * C::WTM + lrow) * TKB + ((((s * C::KB + lane_k(f)) / 16) ^ swz) * 16);
  // B: MS = 16: column block wn*4 + ni, K block s*(KB/64) + f, the lane's 16
  // bytes at 16*lane. MS = 32: lane column lrow lies in block wn*4 + 2ni +
  // lrow/16, row lrow%16 of it; K step s covers K block s/2, groups
  // 2*(s%2) + lgrp.
  uint32_t b_rd0;
  if constexpr (MS == 16)
    b_rd0 = C::ABYTES + (wn * 4) * C::KBLK * 1024 + lane * 16;
  else
    b_rd0 = C::ABYTES + (wn * 4 + lrow / 16) * C::KBLK * 1024 + lgrp * 256 + (lrow % 16) * 16;
  auto b_rd = [&](int s, int ni, int f) -> uint32_t {
    if constexpr (MS == 16) return b_rd0 + (ni * C::KBLK + s * (C::KB / 64) + f) * 1024;
    else return b_rd0 + (2 * ni * C::KBLK + s / 2) * 1024 + (s % 2) * 512;
  };

  // FP8 scales -> LDS before any operand DMA: wave 0 the 256 row scales,
  // wave 1 the 256 column scales (one KiB each).
  if constexpr (DT == DT_FP8) {
    if (wave == 0) lds_dma16((const float*)p.sa + m0, C::TM * 4, lds + C::FSC_OFF, lane * 16);
    if (wave == 1) lds_dma16((const float*)p.sb + n0, C::TN * 4, lds + C::FSC_OFF + C::TM * 4, lane * 16);
  }
  // the fused-epilogue bias (wave 2, one KiB); without one its LDS slot
  // holds zeros (written before the first barrier, read after the last)
  if constexpr (C::BIAS) {
    if (wave == 2) {
      if (p.bias) lds_dma16(p.bias + n0, C::TN * 4, lds + C::BIAS_OFF, lane * 16);
      else *(v4f*)(lds + C::BIAS_OFF + lane * 16) = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }

  Acc acc[C::MREP][C::NACC];
#pragma unroll
  for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NACC; ++ni) acc[mi][ni] = Acc{};

  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // s_waitcnt vmcnt(n) alone
  auto wait_vm = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };

  auto compute = [&](auto st_c, int kn) {
    constexpr int st = decltype(st_c)::value;
    constexpr int sn = (st + C::ST - 1) % C::ST;   // stage of the tile ST-1 ahead
    const char* stage = lds + st * C::STAGE;
    constexpr int NF = C::KSTEPS * C::MREP;
    constexpr int RA = C::RA < NF ? C::RA : NF;
    constexpr int LH = NF > 1 ? NF / 2 : 1;        // fragment groups carrying DMAs
    const int ktn = __builtin_amdgcn_readfirstlane(kn);
    v4i af[RA + 1][C::FRAG];
    v4i bq[2][C::NACC][C::FRAG];
    auto read_b = [&](int s, v4i (*dst)[C::FRAG]) {
#pragma unroll
      for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
        for (int f = 0; f < C::FRAG; ++f) dst[ni][f] = *(const v4i*)(stage + b_rd(s, ni, f));
    };
    auto read_a = [&](int s, int mi, v4i* dst) {
#pragma unroll
      for (int f = 0; f < C::FRAG; ++f) dst[f] = *(const v4i*)(stage + a_rd[s][f] + mi * MS * TKB);
    };
    read_b(0, bq[0]);
#pragma unroll
    for (int j = 0; j < RA; ++j) read_a(j / C::MREP, j % C::MREP, af[j]);
    fence();
    static_for<0, NF>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      constexpr int s = i / C::MREP, mi = i % C::MREP;
      if constexpr (i < LH) {
        static_for<i * C::NVMEM / LH, (i + 1) * C::NVMEM / LH>([&](auto j_c) { dma(sn, ktn, decltype(j_c)::value); });
      }
      if constexpr (mi == 0 && s + 1 < C::KSTEPS) read_b(s + 1, bq[(s + 1) & 1]);
      if constexpr (i + RA < NF) read_a((i + RA) / C::MREP, (i + RA) % C::MREP, af[(i + RA) % (RA + 1)]);
      fence();
#pragma unroll
      for (int ni = 0; ni < C::NACC; ++ni) acc[mi][ni] = mma<DT, MS>(bq[s & 1][ni], af[i % (RA + 1)], acc[mi][ni]);
      fence();
    });
  };

  // tile kt+1's DMAs were issued ST-2 iterations ago: everything issued
  // after them may stay in flight
  using WAIT = std::integral_constant<int, (C::ST - 2) * C::NVMEM>;

  // ---- prologue: tiles 0 .. ST-2 into stages 0 .. ST-2 ----
  static_for<0, C::ST - 1>([&](auto j_c) {
    constexpr int j = decltype(j_c)::value;
    const int kj = __builtin_amdgcn_readfirstlane(min(j, KT - 1));
    static_for<0, C::NVMEM>([&](auto q_c) { dma(j, kj, decltype(q_c)::value); });
  });
  wait_vm(WAIT{});
  __syncthreads();

  // ---- main loop ----
  auto iter = [&](auto r_c, int kt) {
    // past the end the last tile reloads itself into the free stage
    compute(r_c, min(kt + C::ST - 1, KT - 1));
    wait_vm(WAIT{});
    __syncthreads();
  };
  int kt = 0;
  for (; kt + C::ST <= KT; kt += C::ST)
    static_for<0, C::ST>([&](auto r_c) { iter(r_c, kt + decltype(r_c)::value); });
  static_for<0, C::ST - 1>([&](auto r_c) {
    if (kt + decltype(r_c)::value < KT) iter(r_c, kt + decltype(r_c)::value);
  });
  // no DMA may still be writing LDS when the epilogue reuses it
  wait_vm(std::integral_constant<int, 0>{});
  __syncthreads();

  // ---- epilogue ----
  // acc[mi][ni] register 4h + r holds C[wm*WTM + mi*MS + lrow][wn*WTN + ni*MS + col_run(h) + r]
  auto col_run = [&](int h) -> int { return MS == 16 ? 4 * lgrp : 8 * h + 4 * lgrp; };
  const int row0 = wm * C::WTM + lrow;
  const int col0 = wn * C::WTN;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(p.c + ((size_t)m0 * p.N + n0) * C::OB, ((C::TM - 1) * p.N + C::TN) * C::OB);
  // rows / columns an edge tile shares with its neighbour: offset outside the resource
  auto c_off = [&](uint32_t r, uint32_t c) -> uint32_t {
    return (r >= mskip && c >= nskip) ? (r * p.N + c) * C::OB : 0x80000000u;
  };
  float sav[C::MREP];
  v4f sbv[C::NACC][C::NREG / 4];
  if constexpr (DT == DT_FP8) {
    const float* fsa = (const float*)(lds + C::FSC_OFF);
    const float* fsb = fsa + C::TM;
#pragma unroll
    for (int mi = 0; mi < C::MREP; ++mi) sav[mi] = fsa[row0 + mi * MS];
#pragma unroll
    for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
      for (int h = 0; h < C::NREG / 4; ++h) sbv[ni][h] = *(const v4f*)(fsb + col0 + ni * MS + col_run(h));
  }
  // bias of a run of 4 columns (read from LDS where it is used)
  auto bias4 = [&](int ni, int h) -> v4f {
    if constexpr (C::BIAS) return *(const v4f*)(lds + C::BIAS_OFF + (col0 + ni * MS + col_run(h)) * 4);
    else return v4f{0.f, 0.f, 0.f, 0.f};
  };
  if constexpr (!C::CSHUF) {
#pragma unroll
    for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
        for (int h = 0; h < C::NREG / 4; ++h) {
          v4i v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * h + r];
          buf_store16(v, rc, c_off(row0 + mi * MS, col0 + ni * MS + col_run(h)));
        }
  } else {
    auto stage_tile = [&](auto act_c) {
      constexpr int A = decltype(act_c)::value;
#pragma unroll
      for (int mi = 0; mi < C::MREP; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NACC; ++ni)
#pragma unroll
          for (int h = 0; h < C::NREG / 4; ++h) {
            v4f v;
            const v4f bv = bias4(ni, h);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = acc[mi][ni][4 * h + r];
              if constexpr (DT == DT_FP8) x = (x * sav[mi]) * sbv[ni][h][r];
              v[r] = activate<A>(x + bv[r]);
            }
            *(v2i*)(lds + (row0 + mi * MS) * C::CSTRIDE + (col0 + ni * MS + col_run(h)) * C::OB) = pack_out4<DT>(v);
          }
    };
    if constexpr (FUSED) with_act(p.act, stage_tile);
    else stage_tile(std::integral_constant<int, ACT_NONE>{});
    __syncthreads();
    constexpr int CH_ROW = C::TN * C::OB / 16;
    constexpr int TOTAL = C::TM * CH_ROW;
    static_assert(TOTAL % C::THREADS == 0, "whole store passes");
#pragma unroll
    for (int i = 0; i < TOTAL / C::THREADS; ++i) {
      const int q = i * C::THREADS + tid;
      const int row = q / CH_ROW, ch = q % CH_ROW;
      buf_store16(*(const v4i*)(lds + row * C::CSTRIDE + ch * 16), rc, c_off(row, ch * 16 / C::OB));
    }
  }
}

}  // namespace gp
