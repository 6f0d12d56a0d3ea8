// Shared device helpers for the gfx950 preshuffle GEMM kernels.
//
// Vector types, buffer-resource loads/stores, the gfx950 MFMA wrappers for
// each input type, the bf16 / fp16 round-to-nearest-even conversions, the
// fused-epilogue activations and the INT4 widening of the W4A8 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

// On a lambda: inline it at every call. The kernels are written as one body
// of lambdas; left to its own heuristics the compiler may keep a large one
// (the K-tile iteration of the biggest tiles) as a called function, and the
// accumulator array it updates then lives in scratch memory.
#define GP_INLINE __attribute__((always_inline))

namespace gp {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// f(std::integral_constant<int, j>) for j = J0 .. J1-1, unrolled at compile time
template <int J0, class F, int... Js>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Js...>) {
  (f(std::integral_constant<int, J0 + Js>{}), ...);
}
template <int J0, int J1, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<J0>(f, std::make_integer_sequence<int, (J1 > J0 ? J1 - J0 : 0)>{});
}

// DT_I4: int8 A times INT4 B (W4A8); B is widened to int8 in registers and
// multiplied on the int8 instructions.
enum DType : int { DT_I8 = 0, DT_FP8 = 1, DT_BF16 = 2, DT_FP4 = 3, DT_F16 = 4, DT_I4 = 5 };

// Activations of the fused epilogue (values of the C ABI's GP_ACT_*).
enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2, ACT_GELU = 3 };
enum Epi : int { EPI_DIRECT = 1, EPI_CSHUFFLE = 2 };

// gfx9 buffer resource word 3 (32-bit raw buffer, bounds checked on num_records).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ v2i buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ int buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// Loads marked volatile (bit 31 of the aux operand, honoured by the compiler
// only): issued where they stand in program order, never sunk towards their
// first use. For small values needed only at the end of a kernel whose memory
// latency should overlap the main loads.
constexpr int kAuxVolatile = (int)0x80000000u;
__device__ __forceinline__ int buf_load4_early(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kAuxVolatile);
}
__device__ __forceinline__ v4i buf_load16_early(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAuxVolatile);
}
// Global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane
// l's bytes land at LDS byte lds_addr + 16*l. Issued from inline assembly so
// that the compiler does not track the copy: its own tracking cannot tell LDS
// buffers apart and makes the next LDS read wait for every copy in flight,
// which would cap a multi-stage pipeline at one stage of latency. Callers wait
// for the copy with an explicit s_waitcnt vmcnt that counts it in program
// order. The compiler's own vmcnt waits only get stricter from loads it does
// not count, never looser. M0 is set here; no compiler-generated code in these
// kernels uses M0 (LDS instructions on gfx9 and later do not need it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t bytes, const void* lds_dst, uint32_t voff) {
  // buffer resource of [base, base + bytes), every dword made explicitly
  // wave-uniform so that the asm operand can live in SGPRs
  const uint64_t a = (uint64_t)(uintptr_t)base;
  v4i d;
  d[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffff);
  d[2] = (int)__builtin_amdgcn_readfirstlane(bytes);
  d[3] = kRsrcWord3;
  const uint32_t m0v =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff), "s"(d)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Agent-coherent variants: cache policy bit 4 (sc1) on gfx950, the form the
// compiler gives relaxed agent-scope atomic loads and stores. Data written
// this way by one workgroup and read this way by another, on any XCD, needs
// no L2 write-back or invalidate; ordering comes from waiting for the stores
// to complete (s_waitcnt vmcnt(0)) before the atomic that publishes them.
constexpr int kPolicySC1 = 16;
__device__ __forceinline__ v4i buf_load16_coh(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kPolicySC1);
}
__device__ __forceinline__ void buf_store16_coh(v4i v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kPolicySC1);
}

// Non-temporal (streaming) variants: cache policy bit 1 (nt) on gfx950.
constexpr int kPolicyNT = 2;
__device__ __forceinline__ v4i buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicyNT);
}
__device__ __forceinline__ void buf_store16_nt(v4i v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kPolicyNT);
}
__device__ __forceinline__ void buf_store8_nt(v2i v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, kPolicyNT);
}
__device__ __forceinline__ void buf_store16(v4i v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store8(v2i v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}

// The scaled f8f6f4 MFMA with 4-dword (FP4) operands. The clang builtin types
// both sources as 8 dwords, which makes the register allocator reserve 8-VGPR
// tuples for FP4 operands; the LLVM intrinsic is overloaded on the source
// vector type, so it is declared here with 4-dword sources.
__device__ v4f mfma_scale_16x16x128_v4(v4i a, v4i b, v4f c, int cbsz, int blgp, int opsel_a, int scale_a,
                                       int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v4i32");

// Per-type traits. KB = K bytes one MFMA consumes per 16x16 block;
// FRAG = 16-byte pieces per lane per MFMA (1, or 2 for the FP8 K=128 form).
template <int DT> struct Traits;
template <> struct Traits<DT_I8>   { static constexpr int KB = 64;  static constexpr int FRAG = 1; using Acc = v4i; };
template <> struct Traits<DT_BF16> { static constexpr int KB = 64;  static constexpr int FRAG = 1; using Acc = v4f; };
template <> struct Traits<DT_F16>  { static constexpr int KB = 64;  static constexpr int FRAG = 1; using Acc = v4f; };
template <> struct Traits<DT_FP4>  { static constexpr int KB = 64;  static constexpr int FRAG = 1; using Acc = v4f; };
template <> struct Traits<DT_FP8>  { static constexpr int KB = 128; static constexpr int FRAG = 2; using Acc = v4f; };
// W4A8 (small-M kernel only): KB counts bytes of B; one 16-byte INT4 piece
// (32 K elements) feeds two int8 MFMAs.
template <> struct Traits<DT_I4>   { static constexpr int KB = 64;  static constexpr int FRAG = 1; using Acc = v4i; };

// One 16x16 MFMA step. X supplies the first operand (its lane l gives row l%16,
// K piece l/16), Y the second. The result in lane l is D[4*(l/16)+r][l%16].
// sx / sy are the E8M0 block scales of the X / Y lanes (FP4 only).
template <int DT>
__device__ __forceinline__ typename Traits<DT>::Acc
mfma(const v4i* x, const v4i* y, typename Traits<DT>::Acc acc, int sx = 0, int sy = 0) {
  if constexpr (DT == DT_I8) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(x[0], y[0], acc, 0, 0, 0);
  } else if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, x[0]),
                                                   __builtin_bit_cast(v8bf, y[0]), acc, 0, 0, 0);
  } else if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x[0]),
                                                  __builtin_bit_cast(v8h, y[0]), acc, 0, 0, 0);
  } else if constexpr (DT == DT_FP8) {
    v8i xx = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
    v8i yy = __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
    // format 0 = FP8 E4M3 for both operands; constant zero scales select the
    // unscaled 16x16x128 f8f6f4 instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xx, yy, acc, 0, 0, 0, 0, 0, 0);
  } else {
    // format 4 = FP4 E2M1 for both operands; byte 0 of sx / sy is the E8M0 scale.
    return mfma_scale_16x16x128_v4(x[0], y[0], acc, 4, 4, 0, sx, 0, sy);
  }
}

// FP4 MFMA whose E8M0 scales sit in byte SEL of sx / sy (op_sel picks the byte).
template <int SEL>
__device__ __forceinline__ v4f mfma_fp4_sel(const v4i* x, const v4i* y, v4f acc, int sx, int sy) {
  return mfma_scale_16x16x128_v4(x[0], y[0], acc, 4, 4, SEL, sx, SEL, sy);
}

__device__ v16f mfma_scale_32x32x64_v4(v4i a, v4i b, v16f c, int cbsz, int blgp, int opsel_a, int scale_a,
                                       int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");

// MFMA shape: MS x MS output block per instruction.
//   MS = 16: lane l supplies row/column l%16 and the 16-byte K piece(s) of
//            lane group l/16; result D[4*(l/16)+r][l%16] in 4 registers.
//   MS = 32: lane l supplies row/column l%32 and the 16-byte K piece of lane
//            group l/32; result D[8*i+4*(l/32)+j][l%32] in register 4*i+j.
// A 32x32 form (BF16 32x32x16, FP4 32x32x64, ...) does twice the FLOPs of
// the 16x16 form per instruction and reads fewer operand bytes per FLOP; the
// counters show 16 issue cycles per BF16 16x16x32 and 32 per FP8 16x16x128.
template <int DT, int MS> struct Mma;
template <int DT> struct Mma<DT, 16> {
  static constexpr int KB = Traits<DT>::KB;     // K bytes per instruction
  static constexpr int FRAG = Traits<DT>::FRAG; // 16-byte pieces per lane
  static constexpr int NREG = 4;                // result registers per lane
  using Acc = typename Traits<DT>::Acc;
};
template <int DT> struct Mma<DT, 32> {
  static_assert(DT != DT_FP8, "FP8 uses the 16x16x128 instruction");
  static constexpr int KB = 32;
  static constexpr int FRAG = 1;
  static constexpr int NREG = 16;
  using Acc = std::conditional_t<DT == DT_I8, v16i, v16f>;
};

// One MS x MS MFMA. X is the first operand, Y the second; FP4 scales sx / sy
// sit in byte SEL of their registers.
template <int DT, int MS, int SEL = 0>
__device__ __forceinline__ typename Mma<DT, MS>::Acc mma(const v4i* x, const v4i* y, typename Mma<DT, MS>::Acc acc,
                                                         int sx = 0, int sy = 0) {
  if constexpr (MS == 16) {
    if constexpr (DT == DT_FP4) return mfma_scale_16x16x128_v4(x[0], y[0], acc, 4, 4, SEL, sx, SEL, sy);
    else return mfma<DT>(x, y, acc);
  } else {
    if constexpr (DT == DT_I8) {
      return __builtin_amdgcn_mfma_i32_32x32x32_i8(x[0], y[0], acc, 0, 0, 0);
    } else if constexpr (DT == DT_BF16) {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, x[0]), __builtin_bit_cast(v8bf, y[0]), acc,
                                                     0, 0, 0);
    } else if constexpr (DT == DT_F16) {
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, x[0]), __builtin_bit_cast(v8h, y[0]), acc,
                                                    0, 0, 0);
    } else {
      return mfma_scale_32x32x64_v4(x[0], y[0], acc, 4, 4, SEL, sx, SEL, sy);
    }
  }
}

// fp32 -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// fp32 -> fp16 with round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  _Float16 a = (_Float16)lo;
  _Float16 b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Four fp32 results -> 8 bytes of the output type.
template <int DT>
__device__ __forceinline__ v2i pack_out4(v4f v) {
  v2i o;
  if constexpr (DT == DT_F16) {
    o[0] = (int)pack_f16x2(v[0], v[1]);
    o[1] = (int)pack_f16x2(v[2], v[3]);
  } else {
    o[0] = (int)pack_bf16x2(v[0], v[1]);
    o[1] = (int)pack_bf16x2(v[2], v[3]);
  }
  return o;
}

// erf for the GELU epilogue: Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26, erf(x) = 1 - (a1 t + ... + a5 t^5) e^(-x^2),
// t = 1 / (1 + p x), for x >= 0 (absolute error <= 1.5e-7, well below the
// bf16 / fp16 output rounding), odd symmetry for x < 0. About 15 VALU
// operations, a fraction of a library erf, which matters where the epilogue
// sits on the critical path (the small-M kernel).
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return copysignf(1.f - poly * __expf(-ax * ax), x);
}

// The value of x, hidden from the optimizer: every quantity derived from the
// result is computed where this call stands. Used at the start of epilogues
// so that their per-lane addresses are not hoisted above the K loop, where
// they would occupy registers through it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Fused epilogue activation (Kernel Tuning Guide §6: bias, bias+ReLU,
// bias+SiLU, bias+GELU), chosen at compile time; with_act() dispatches a
// kernel's uniform `act` once, so no per-element branch is left.
//   relu(x) = max(x, 0); silu(x) = x / (1 + e^-x); gelu(x) = x/2 (1 + erf(x / sqrt 2)).
// The reciprocal is the hardware's (1 ulp), again far below the output rounding.
template <int A>
__device__ __forceinline__ float activate(float x) {
  if constexpr (A == ACT_RELU) return fmaxf(x, 0.f);
  else if constexpr (A == ACT_SILU) return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
  else if constexpr (A == ACT_GELU) return 0.5f * x * (1.f + erf_as7126(x * 0.70710678118654752f));
  else return x;
}
template <class F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(std::integral_constant<int, ACT_RELU>{}); break;
    case ACT_SILU: f(std::integral_constant<int, ACT_SILU>{}); break;
    case ACT_GELU: f(std::integral_constant<int, ACT_GELU>{}); break;
    default: f(std::integral_constant<int, ACT_NONE>{}); break;
  }
}

// W4A8: one 16-byte piece of the INT4 layout holds 32 K elements of a
// column, elements 0..15 in the low nibbles and 16..31 in the high nibbles
// of its 16 bytes. Widening keeps each nibble in the top half of its byte,
// i.e. the int8 value 16 * v: two masks (and a shift) per dword, and the
// int8 products come out exactly 16 times too large (undone in the epilogue).
__device__ __forceinline__ void widen_int4(v4i w, v4i& lo, v4i& hi) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    lo[d] = (int)(((uint32_t)w[d] << 4) & 0xF0F0F0F0u);
    hi[d] = (int)((uint32_t)w[d] & 0xF0F0F0F0u);
  }
}

}  // namespace gp
