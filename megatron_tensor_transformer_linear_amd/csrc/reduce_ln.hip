// Partial reduce + residual + LayerNorm, the in-HBM replacement of the tensor-parallel
// all-reduce (pwwt.cn TP walk-through section 2.3: the all-reduce sits just before the
// residual add and can be fused with it and with the next LayerNorm's statistics; section
// 6.3: residual + LayerNorm as one fused op with one fixed statistics order).
//
//   h = residual + sum_{p ascending} parts[p];  y = (h - mean) / sqrt(var + eps) * gamma + beta
//
// HBM-bound: one workgroup per row streams every partial once (16-byte loads, coalesced
// along the row), keeps the row in registers, and writes h and y once.  Row statistics are
// a wave reduction (cross-lane shuffles) followed by a cross-wave step through LDS; the
// variance is the second pass over the register-resident row (no E[x^2] - mean^2).
#include "common.hpp"

namespace tpk {
namespace {

template <int THREADS>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < THREADS / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* p, int64_t idx) {
  if (BF16) {
    const uint2 u = *(const uint2*)((const bf16_t*)p + idx);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
  } else {
    return *(const float4*)((const float*)p + idx);
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* p, int64_t idx, float4 v) {
  if (BF16) {
    uint2 u;
    u.x = pack_bf16x2(v.x, v.y);
    u.y = pack_bf16x2(v.z, v.w);
    *(uint2*)((bf16_t*)p + idx) = u;
  } else {
    *(float4*)((float*)p + idx) = v;
  }
}

template <int THREADS, int VPT, bool BF16>
__global__ __launch_bounds__(THREADS) void reduce_ln_kernel(ReduceDesc r) {
  __shared__ float red[THREADS / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t H = r.H;
  const int64_t roff = row * H;

  float4 v[VPT];
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int64_t col = ((int64_t)c * THREADS + tid) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < H) {
      if (r.n_parts > 0) {
        acc = *(const float4*)(r.parts + roff + col);
        for (int p = 1; p < r.n_parts; ++p) {
          const float4 q = *(const float4*)(r.parts + (int64_t)p * r.part_stride + roff + col);
          acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
        }
      }
      if (r.residual) {
        const float4 q = load4<BF16>(r.residual, roff + col);
        acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
      }
      if (r.h_out) store4<BF16>(r.h_out, roff + col, acc);
    }
    v[c] = acc;
    sum += (acc.x + acc.y) + (acc.z + acc.w);
  }
  if (!r.gamma) return;

  const float inv_h = 1.0f / (float)H;
  const float mean = block_sum<THREADS>(sum, red) * inv_h;
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int64_t col = ((int64_t)c * THREADS + tid) * 4;
    if (col < H) {
      const float a0 = v[c].x - mean, a1 = v[c].y - mean, a2 = v[c].z - mean, a3 = v[c].w - mean;
      sq += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float var = block_sum<THREADS>(sq, red) * inv_h;
  const float rstd = 1.0f / sqrtf(var + r.eps);
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int64_t col = ((int64_t)c * THREADS + tid) * 4;
    if (col < H) {
      const float4 g = load4<BF16>(r.gamma, col);
      float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r.beta) b = load4<BF16>(r.beta, col);
      float4 y;
      y.x = (v[c].x - mean) * rstd * g.x + b.x;
      y.y = (v[c].y - mean) * rstd * g.y + b.y;
      y.z = (v[c].z - mean) * rstd * g.z + b.z;
      y.w = (v[c].w - mean) * rstd * g.w + b.w;
      store4<BF16>(r.y_out, roff + col, y);
    }
  }
}

template <int THREADS, int VPT>
hipError_t launch_t(const ReduceDesc& r, hipStream_t stream) {
  dim3 grid((unsigned)r.rows), block(THREADS);
  if (r.bf16)
    hipLaunchKernelGGL((reduce_ln_kernel<THREADS, VPT, true>), grid, block, 0, stream, r);
  else
    hipLaunchKernelGGL((reduce_ln_kernel<THREADS, VPT, false>), grid, block, 0, stream, r);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_ln(const ReduceDesc& r, hipStream_t stream) {
  if (r.rows <= 0) return hipSuccess;
  if (r.rows > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t h4 = (r.H + 3) / 4;
  if (h4 <= 256 * 1) return launch_t<256, 1>(r, stream);
  if (h4 <= 256 * 2) return launch_t<256, 2>(r, stream);
  if (h4 <= 256 * 3) return launch_t<256, 3>(r, stream);
  if (h4 <= 256 * 4) return launch_t<256, 4>(r, stream);
  if (h4 <= 256 * 6) return launch_t<256, 6>(r, stream);
  if (h4 <= 256 * 8) return launch_t<256, 8>(r, stream);
  if (h4 <= 256 * 12) return launch_t<256, 12>(r, stream);
  if (h4 <= 256 * 16) return launch_t<256, 16>(r, stream);
  if (h4 <= 1024 * 8) return launch_t<1024, 8>(r, stream);
  if (h4 <= 1024 * 16) return launch_t<1024, 16>(r, stream);
  return hipErrorInvalidValue;
}

}  // namespace tpk
