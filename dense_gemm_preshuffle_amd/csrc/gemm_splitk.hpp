// Small-M preshuffle GEMM kernel (memory-bound regime) for gfx950.
//
// For M of a few 16-row blocks the GEMM is bound by streaming B from HBM
// (Kernel Tuning Guide §0 "Is the kernel memory-, compute-, or
// latency-bound?", GEMM Optimization Guide §8.3). The pages' small-batch tile
// (16 x 64-128 x 256-512, §1.3) walks K sequentially in one workgroup, which
// leaves few workgroups and few bytes in flight per CU. Here a workgroup owns
// 16 rows x (16*NB) columns and its WAVES waves split K: each wave issues the
// loads for its whole K range up front (in chunks of KCH bytes, the next
// chunk's loads issued before the current chunk's MFMAs), so that most of B
// is in flight at once. Partial sums are reduced through LDS in a fixed order
// (deterministic), then scaled, biased, activated, rounded and stored.
//
// Operands come straight from global memory in MFMA layout: B from the
// preshuffled layout (one KiB per 16 columns x 64 K bytes), A as 16 bytes per
// lane (row lane%16, K piece lane/16), which is L2-resident since every
// workgroup reads the same few rows. B is read exactly once, so its loads and
// the C stores carry the non-temporal cache policy and leave L2 to A.
//
// M needs no particular multiple: the last 16-row block reads its missing
// rows of A (and of the FP8 / W4A8 row scales, FP4 block scales) as zeros
// through the bounds of its buffer resources and stores only its real rows.
//
// W4A8 (DT_I4): each 16-byte piece of the INT4 B layout holds K elements
// 0..15 of the piece in its low nibbles and 16..31 in its high nibbles; it is
// widened to two int8 operands (16 x the value, see widen_int4) and
// multiplied with the matching two 16-byte pieces of the int8 A row.
#pragma once

#include <type_traits>

#include "gp_common.hpp"

namespace gp {

struct SplitArgs {
  const char* a;
  const char* b;
  const void* sa;
  const void* sb;
  const float* bias;  // fp32 [N] or null (fused epilogue)
  char* c;
  uint32_t M, N, Kb;  // Kb = bytes per row of B (A rows are 2 Kb bytes for W4A8)
  int act;            // Act
};

// MB: 16-row blocks per workgroup (1 for M = 16; up to 4 so that a batch of
// up to 64 rows reads B once); each wave multiplies every block of its K range.
template <int DT, int NB, int WAVES, int KCH, int MB = 1>
struct SplitCfg {
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KB = Traits<DT>::KB;
  static constexpr int FRAG = Traits<DT>::FRAG;
  static constexpr int STEPS = KCH / KB;              // B pieces (K steps) per chunk
  static constexpr int AW = (DT == DT_I4) ? 2 : 1;    // A bytes per B byte
  static constexpr int AFR = FRAG * AW;               // A pieces per lane per step
  static constexpr int OB = (DT == DT_I8) ? 4 : 2;
  static constexpr int NSC = (DT == DT_FP4) ? 1 : 0;
  static constexpr bool FSC = DT == DT_FP8 || DT == DT_I4;   // fp32 row / column scales
  static constexpr int NQ = MB * NB;                  // 16 x 16 output blocks
  static constexpr int LDS = WAVES * NQ * 64 * 16;    // partial accumulators
  static_assert(KCH % KB == 0, "chunk must be whole MFMA steps");
  static_assert(NQ <= WAVES, "one output block per wave in the epilogue");
};

template <int DT, int NB, int WAVES, int KCH, int MB>
__global__ __launch_bounds__(WAVES * 64) void gemm_splitk_kernel(SplitArgs p) {
  using C = SplitCfg<DT, NB, WAVES, KCH, MB>;
  using Acc = typename Traits<DT>::Acc;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];

  const int tid = threadIdx.x;
  // wave index: uniform across the wave; readfirstlane puts it in a scalar
  // register so that offsets derived from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lane_lo = lane & 15;
  const int lane_hi = lane >> 4;

  const uint32_t Kb = p.Kb;
  const uint32_t Ka = Kb * C::AW;           // bytes per row of A
  // Column tiles go round-robin to the 8 XCDs; remap so that each XCD owns a
  // contiguous run of tiles. Neighbouring tiles then share whole 128-byte
  // lines of C inside one XCD's L2 instead of writing halves from two XCDs.
  uint32_t bx = blockIdx.x;
  if (gridDim.x % 8u == 0) bx = (bx % 8u) * (gridDim.x / 8u) + bx / 8u;
  const uint32_t n0 = bx * (16 * NB);
  const uint32_t m0 = blockIdx.y * (16 * MB);
  const uint32_t mrows = min(16u * MB, p.M - m0);  // real rows of this workgroup
  const uint32_t kw = Kb / WAVES;            // B bytes per wave
  const uint32_t k_begin = wave * kw;
  const int chunks = (int)(kw / KCH);

  // A resource covers the block's real rows only; the row is always part of
  // the per-lane offset, so a missing row reads zeros without a memory access.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * Ka, mrows * Ka);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * Kb, 16 * NB * Kb);
  // W4A8: the B piece of lane group g covers K elements [32g, 32g+32) of a
  // 128-element block, i.e. A bytes 32g + 16h for its two halves h
  const uint32_t a_off = lane_lo * Ka + lane_hi * 16 * C::AW;
  uint32_t b_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b_off[nb] = nb * 16 * Kb + lane * 16;

  const uint32_t srow = Kb / 16;
  __amdgpu_buffer_rsrc_t rsa = make_rsrc(nullptr, 0), rsb = make_rsrc(nullptr, 0);
  if constexpr (DT == DT_FP4) {
    rsa = make_rsrc((const char*)p.sa + (size_t)m0 * srow, mrows * srow);
    rsb = make_rsrc((const char*)p.sb + (size_t)n0 * srow, 16 * NB * srow);
  }

  // Epilogue vectors (row / column scales, bias): issued before any operand
  // load, so that the epilogue does not wait one more memory round trip for
  // them. Wave w stores output block w = (row block w / NB, column block
  // w % NB), so each wave needs its block's row and column values only.
  const uint32_t qw = (uint32_t)min(wave, C::NQ - 1);
  const uint32_t nbw = qw % NB, mbw = qw / NB;
  float sa_v = 1.f;
  v4f sb_v = v4f{1.f, 1.f, 1.f, 1.f};
  if constexpr (C::FSC) {
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc((const float*)p.sa + m0, mrows * 4);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc((const float*)p.sb + n0, 16 * NB * 4);
    sa_v = __builtin_bit_cast(float, buf_load4_early(rs_a, (mbw * 16 + lane_lo) * 4, 0));
    sb_v = __builtin_bit_cast(v4f, buf_load16_early(rs_b, (nbw * 16 + 4 * lane_hi) * 4, 0));
  }
  // without a bias the resource is empty: the load returns zeros, no branch
  v4f bias_v = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (DT != DT_I8) {
    const bool has_bias = p.bias != nullptr;
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(has_bias ? p.bias + n0 : p.bias, has_bias ? 16 * NB * 4 : 0);
    bias_v = __builtin_bit_cast(v4f, buf_load16_early(rbias, (nbw * 16 + 4 * lane_hi) * 4, 0));
  }

  v4i af[2][C::STEPS][MB][C::AFR];
  v4i bf[2][C::STEPS][NB][C::FRAG];
  int sa_r[2][C::STEPS][MB * C::NSC + 1 - C::NSC];
  int sb_r[2][C::STEPS][NB * C::NSC + 1 - C::NSC];
  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Acc{0, 0, 0, 0};

  auto load = [&](auto par_c, int ch) {
    constexpr int par = decltype(par_c)::value;
    const uint32_t kb = k_begin + (uint32_t)ch * KCH;  // B byte of this chunk
#pragma unroll
    for (int s = 0; s < C::STEPS; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int f = 0; f < C::AFR; ++f) {
          const uint32_t ao = a_off + mb * 16 * Ka;
          if constexpr (DT == DT_I4) af[par][s][mb][f] = buf_load16(ra, ao + s * 128 + f * 16, kb * 2);
          else af[par][s][mb][f] = buf_load16(ra, ao + s * C::KB + f * 64, kb);
        }
    const uint32_t kblk = (kb / 64) * 1024u;
#pragma unroll
    for (int s = 0; s < C::STEPS; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int f = 0; f < C::FRAG; ++f)
          bf[par][s][nb][f] = buf_load16_nt(rb, b_off[nb] + (s * (C::KB / 64) + f) * 1024, kblk);
    if constexpr (DT == DT_FP4) {
      const uint32_t sbase = kb / 16;  // scale byte of this chunk's first 32-element block
#pragma unroll
      for (int s = 0; s < C::STEPS; ++s) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sa_r[par][s][mb] = buf_load4(rsa, (mb * 16 + lane_lo) * srow + s * 4, sbase);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sb_r[par][s][nb] = buf_load4(rsb, (nb * 16 + lane_lo) * srow + s * 4, sbase);
      }
    }
  };
  auto compute = [&](auto par_c) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int s = 0; s < C::STEPS; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // W4A8: the piece is widened once and used by every row block
        v4i lo, hi;
        if constexpr (DT == DT_I4) widen_int4(bf[par][s][nb][0], lo, hi);
        int sx = 0;
        if constexpr (DT == DT_FP4) sx = sb_r[par][s][nb] >> (8 * lane_hi);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (DT == DT_I4) {
            acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo, af[par][s][mb][0], acc[mb][nb], 0, 0, 0);
            acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi, af[par][s][mb][1], acc[mb][nb], 0, 0, 0);
          } else {
            int sy = 0;
            if constexpr (DT == DT_FP4) sy = sa_r[par][s][mb] >> (8 * lane_hi);
            acc[mb][nb] = mfma<DT>(bf[par][s][nb], af[par][s][mb], acc[mb][nb], sx, sy);
          }
        }
      }
    }
  };

  load(std::integral_constant<int, 0>{}, 0);
  int ch = 0;
  for (; ch + 2 <= chunks; ch += 2) {
    load(std::integral_constant<int, 1>{}, ch + 1);
    compute(std::integral_constant<int, 0>{});
    if (ch + 2 < chunks) load(std::integral_constant<int, 0>{}, ch + 2);
    compute(std::integral_constant<int, 1>{});
  }
  if (ch < chunks) compute(std::integral_constant<int, 0>{});

  // ---- reduce the WAVES partial sums through LDS in wave order ----
  Acc* red = (Acc*)lds;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wave * C::NQ + mb * NB + nb) * 64 + lane] = acc[mb][nb];
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(p.c + ((size_t)m0 * p.N + n0) * C::OB, ((mrows - 1) * p.N + 16 * NB) * C::OB);
  with_act(p.act, [&](auto act_c) {
    constexpr int A = decltype(act_c)::value;
    if (wave < C::NQ) {
      Acc v = red[wave * 64 + lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red[(w * C::NQ + wave) * 64 + lane];
      // lane holds C[m0 + mbw*16 + lane_lo][n0 + nbw*16 + 4*lane_hi + r]; rows
      // past M are not stored (offset outside the resource)
      const uint32_t row = mbw * 16 + lane_lo;
      const uint32_t col = nbw * 16 + 4 * lane_hi;
      const uint32_t off = row < mrows ? (row * p.N + col) * C::OB : 0x80000000u;
      if constexpr (DT == DT_I8) {
        buf_store16_nt(v, rc, off);
      } else {
        v4f x;
        if constexpr (DT == DT_I4) {
          // the widened products are 16 x the INT4 ones (exact multiples of 16)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = (float)(v[r] >> 4);
        } else {
          x = v;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = x[r];
          if constexpr (C::FSC) y = (y * sa_v) * sb_v[r];
          x[r] = activate<A>(y + bias_v[r]);
        }
        buf_store8_nt(pack_out4<DT>(x), rc, off);
      }
    }
  });
}

}  // namespace gp
