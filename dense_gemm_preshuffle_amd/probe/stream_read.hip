// HBM streaming-read probe: the floor under the memory-bound GEMM shapes.
//
// The small-batch GEMM is bound by reading B once from HBM (Kernel Tuning
// Guide §0, "Is the kernel memory-, compute-, or latency-bound?"; GEMM
// Optimization Guide §8.3). This kernel does nothing but that read: each of
// `wgs` workgroups streams its contiguous share of a buffer with 16-byte
// non-temporal buffer loads (the load form of the small-M GEMM kernel), all
// of a thread's loads issued before any is used, and folds the data into
// one word per thread so that no load is dead. Its time for the bytes a GEMM
// must read is the floor that GEMM's kernel can approach: what one pass over
// that many bytes costs on this part, first-byte latency and dispatch
// included.
//
// C ABI (used by bench.py --floor; not part of the GEMM library):
//   int gp_probe_stream_read(const void* buf, uint64_t bytes, int wgs, int waves,
//                            uint32_t* sink, void* stream)
//     buf    device, bytes readable, 16-byte aligned; bytes a multiple of
//            16 * 64 * waves * wgs (every lane reads whole 16-byte pieces)
//     wgs    workgroups (1 .. 4096); waves per workgroup 1 .. 16
//     sink   device, wgs * waves * 64 uint32 written (one per thread)
//   Returns 0, or 1 for invalid arguments, 5 for a HIP launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// U loads in flight per thread per batch
constexpr int U = 16;

__global__ __launch_bounds__(1024) void stream_read_kernel(const char* __restrict__ buf, uint32_t per_wg,
                                                           uint32_t* __restrict__ sink) {
  const uint32_t threads = blockDim.x;
  const __amdgpu_buffer_rsrc_t r = rsrc(buf + (size_t)blockIdx.x * per_wg, per_wg);
  v4i acc = {0, 0, 0, 0};
  const uint32_t step = threads * 16u;
  for (uint32_t base = threadIdx.x * 16u; base < per_wg; base += step * U) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + u * step, 0, 2);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  sink[blockIdx.x * threads + threadIdx.x] = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

}  // namespace

extern "C" int gp_probe_stream_read(const void* buf, uint64_t bytes, int wgs, int waves, uint32_t* sink,
                                    void* stream) {
  if (!buf || !sink || wgs < 1 || wgs > 4096 || waves < 1 || waves > 16) return 1;
  if (((uintptr_t)buf & 15u) != 0) return 1;
  const uint64_t unit = 16ull * 64 * waves * wgs;
  if (bytes == 0 || bytes % unit || bytes / wgs >= (1ull << 31)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_read_kernel, dim3(wgs), dim3(64 * waves), 0, (hipStream_t)stream, (const char*)buf,
                     (uint32_t)(bytes / wgs), sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
