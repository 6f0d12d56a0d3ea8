// MFMA issue-rate probe: what each matrix instruction the GEMM kernels use
// sustains on its own.
//
// The Kernel Tuning Guide (§0, "Background: The GPU Performance Model") puts
// MFMA latency at tens of cycles and treats the hot loop's job as keeping the
// matrix pipes fed; the Kernel Bottleneck Tuning page (§1) measures an
// instruction's throughput in isolation on several independent dependency
// chains before tuning a kernel around it. Here every wave runs `iters`
// rounds of 8 MFMAs of one form on 8 independent accumulators, with operands
// in registers and no memory traffic, between two reads of the shader clock
// counter (s_memtime) and of the 100 MHz real-time counter (s_memrealtime).
// Cycles per MFMA per wave, against the instruction's issue cycles, show how
// close a kernel built from that form can get to the dtype's dense peak with
// one (256 workgroups of 4 waves) or two (512) waves per SIMD.
//
// C ABI (used by bench.py --mfma-rate; not part of the GEMM library):
//   int gp_probe_mfma_rate(int form, float* out, unsigned long long* cycles,
//                          int iters, int wgs, void* stream)
//     form    0 bf16 16x16x32, 1 f16 16x16x32, 2 i8 16x16x64, 3 fp8 16x16x128,
//             4 fp4 16x16x128 (scaled), 5 bf16 32x32x16, 6 f16 32x32x16,
//             7 i8 32x32x32, 8 fp8 32x32x64, 9 fp4 32x32x64 (scaled)
//     out     device, wgs * 256 floats written (a checksum per thread)
//     cycles  device, wgs * 4 * 2 uint64 written: per wave, shader-clock
//             cycles and 100 MHz ticks of its timed loop
//     iters   1 .. 1 000 000; wgs 1 .. 4096 (256 threads each)
//   Returns 0, 1 for invalid arguments (checked before any HIP call), 5 for
//   a HIP launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// the scaled FP4 forms with 4-dword sources, as the GEMM kernels issue them
__device__ v4f scale16(v4i a, v4i b, v4f c, int cbsz, int blgp, int oa, int sa, int ob, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v4i32");
__device__ v16f scale32(v4i a, v4i b, v16f c, int cbsz, int blgp, int oa, int sa, int ob, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");

template <int F, typename Acc>
__device__ __forceinline__ Acc step(v4i a, v4i b, Acc c) {
  const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (F == 0) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  if constexpr (F == 1) return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  if constexpr (F == 2) return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  if constexpr (F == 3) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 0, 0, 0, 0, 0, 0);
  if constexpr (F == 4) return scale16(a, b, c, 4, 4, 0, 127, 0, 127);
  if constexpr (F == 5) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  if constexpr (F == 6) return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  if constexpr (F == 7) return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  if constexpr (F == 8) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 0, 0, 0, 0, 0, 0);
  if constexpr (F == 9) return scale32(a, b, c, 4, 4, 0, 127, 0, 127);
}

template <int F, typename Acc, int NR>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* __restrict__ out, unsigned long long* __restrict__ cyc,
                                                        int iters) {
  const int t = threadIdx.x;
  // small integer codes: valid finite values in every input format
  const v4i a = v4i{t, t * 3, t * 5, t * 7} & 0x07070707;
  const v4i b = v4i{t * 11, t * 13, t + 1, t + 2} & 0x07070707;
  Acc c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  __builtin_amdgcn_s_barrier();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = step<F>(a, b, c0);
    c1 = step<F>(a, b, c1);
    c2 = step<F>(a, b, c2);
    c3 = step<F>(a, b, c3);
    c4 = step<F>(a, b, c4);
    c5 = step<F>(a, b, c5);
    c6 = step<F>(a, b, c6);
    c7 = step<F>(a, b, c7);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const Acc s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) sum += (float)s[r];
  out[blockIdx.x * 256 + t] = sum;
  if ((t & 63) == 0) {
    const int w = blockIdx.x * 4 + (t >> 6);
    cyc[2 * w] = t1 - t0;
    cyc[2 * w + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int gp_probe_mfma_rate(int form, float* out, unsigned long long* cyc, int iters, int wgs, void* stream) {
  if (form < 0 || form > 9 || !out || !cyc || iters < 1 || iters > 1000000 || wgs < 1 || wgs > 4096) return 1;
  const dim3 g(wgs), b(256);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  switch (form) {
    case 0: hipLaunchKernelGGL((mfma_rate_kernel<0, v4f, 4>), g, b, 0, s, out, cyc, iters); break;
    case 1: hipLaunchKernelGGL((mfma_rate_kernel<1, v4f, 4>), g, b, 0, s, out, cyc, iters); break;
    case 2: hipLaunchKernelGGL((mfma_rate_kernel<2, v4i, 4>), g, b, 0, s, out, cyc, iters); break;
    case 3: hipLaunchKernelGGL((mfma_rate_kernel<3, v4f, 4>), g, b, 0, s, out, cyc, iters); break;
    case 4: hipLaunchKernelGGL((mfma_rate_kernel<4, v4f, 4>), g, b, 0, s, out, cyc, iters); break;
    case 5: hipLaunchKernelGGL((mfma_rate_kernel<5, v16f, 16>), g, b, 0, s, out, cyc, iters); break;
    case 6: hipLaunchKernelGGL((mfma_rate_kernel<6, v16f, 16>), g, b, 0, s, out, cyc, iters); break;
    case 7: hipLaunchKernelGGL((mfma_rate_kernel<7, v16i, 16>), g, b, 0, s, out, cyc, iters); break;
    case 8: hipLaunchKernelGGL((mfma_rate_kernel<8, v16f, 16>), g, b, 0, s, out, cyc, iters); break;
    default: hipLaunchKernelGGL((mfma_rate_kernel<9, v16f, 16>), g, b, 0, s, out, cyc, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
