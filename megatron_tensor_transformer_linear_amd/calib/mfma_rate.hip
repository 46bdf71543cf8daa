// Calibration kernel (not part of the layer's computation): the matrix-core rate this device
// sustains on its own, used to put the GEMMs' measured rates in context.
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on four independent accumulators,
// touching no memory inside the loop.  Each lane holds eight A and eight B fragments, taken
// from two caller buffers (the workload's own operands), and the MFMAs rotate through them.
// Under a socket power limit the clock, and with it this rate, depends on the operands' bit
// activity (all-zero operands run about 35 % faster than random ones, and two different
// pseudo-random fillings differed by 20 %), so the operands are the real data.  A GEMM on
// those operands cannot exceed this rate on the same device in the same power state.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// Fragment f of lane t: 16 bytes at a 16-byte-aligned offset inside a buffer of `bytes`
// bytes (a multiple of 16), spread over the buffer.
__device__ __forceinline__ bf16x8_t fragment(const char* src, uint64_t bytes, uint64_t idx) {
  const uint64_t chunks = bytes / 16;
  return *(const bf16x8_t*)(src + ((idx * 40503u) % chunks) * 16);
}

__global__ __launch_bounds__(256) void mfma_rate_kernel(const char* asrc, const char* bsrc,
                                                        uint64_t bytes, float* out, int iters) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    a[f] = fragment(asrc, bytes, (uint64_t)t * 8 + f);
    b[f] = fragment(bsrc, bytes, (uint64_t)t * 8 + f + 3);
  }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int f = 0; f < 8; ++f)
      acc[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f], b[(f + 3) & 7], acc[f & 3], 0, 0, 0);
#pragma unroll
    for (int f = 0; f < 8; ++f)
      acc[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(f + 5) & 7], b[f], acc[f & 3], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[t] = s;  // keeps the products live; t < blocks * 256, the size of out
}

}  // namespace

extern "C" {

// Launch `blocks` workgroups of 256 threads, each wave running `iters` rounds of 16 MFMAs
// (32768 flops each) on stream `stream`.  `a_src` and `b_src` are device buffers of `bytes`
// bytes each (16-byte aligned, bytes a positive multiple of 16) whose bf16 contents supply
// the operands; `out` is device memory of blocks * 256 floats.  Returns 0, -1 for invalid
// arguments (nothing launched), or the HIP error of the launch.
int tp_calib_mfma_loop(const void* a_src, const void* b_src, uint64_t bytes, float* out,
                       int blocks, int iters, void* stream) {
  if (!a_src || !b_src || !out || blocks <= 0 || iters <= 0) return -1;
  if (bytes < 16 || bytes % 16 || ((uintptr_t)a_src | (uintptr_t)b_src) % 16) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const char*)a_src, (const char*)b_src, bytes, out, iters);
  return (int)hipGetLastError();
}

// Flops of one such launch.
double tp_calib_mfma_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * (double)iters * 16.0 * 32768.0;
}

}  // extern "C"
