// fp32 MFMA GEMM tile for gfx950 (io dtype fp32): the column / row-parallel linears of the
// small fp32 MLP.  Same contract and epilogues as the bf16 tile (0539edu.com TP tutorial
// section 1.1, formula 1.1 and figure 1.2), built on v_mfma_f32_16x16x4_f32.
//
// Tile 64 x 64 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave 32 x 32 as 2 x 2 blocks
// of 16 x 16.  Operand layout of the 16x16x4 instruction: A lane l holds A[l % 16][l / 16],
// B lane l holds B[l / 16][l % 16]; accumulator element r of lane l is C[4 (l / 16) + r][l % 16].
// These fp32 shapes are a few MFLOP with few tiles, so the time is the chain of K steps: each
// step's global loads go out before the previous step is multiplied (held in registers), and
// the K step is 64 wide so a contraction of 512 takes 8 round trips to memory, not 32.
#include "common.hpp"

namespace tpk {
namespace {

constexpr int TM = 64, TN = 64, TK = 64;
constexpr int NT = 256;

template <int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(GemmDesc g) {
  __shared__ float As[TM][TK + 1];
  __shared__ __attribute__((aligned(16))) float Bs[TK][TN + 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t M = g.M, N = g.N, K = g.K;
  // Tiles are numbered n-fastest over a one-dimensional grid that loops over them, so no size
  // that passes validation exceeds a grid dimension.
  const int64_t tn = (N + TN - 1) / TN, ntiles = ((M + TM - 1) / TM) * tn;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t m0 = (tile / tn) * TM, n0 = (tile % tn) * TN;
    const float* __restrict__ A = (const float*)g.A;
    const float* __restrict__ B = (const float*)g.B;

    // A tile: thread -> rows tid/16 + 16 i, k chunk (tid%16)*4.  B tile: k-rows tid/16 + 16 i,
    // n chunk (tid%16)*4 (i = 0..3).
    const int a_r = tid >> 4, a_k = (tid & 15) * 4;
    const int b_r = tid >> 4, b_n = (tid & 15) * 4;
    const int64_t b_nlog = n0 + b_n;
    const bool b_nvalid = b_nlog < N;
    const int64_t b_col = (b_nlog / g.b_blk) * g.b_blk_stride + (b_nlog % g.b_blk);

    f32x4_t acc[2][2];
  #pragma unroll
    for (int i = 0; i < 2; ++i)
  #pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    float4 ra[4], rb[4];  // the next K step's operands, in flight while the current is multiplied
    auto gload = [&](int64_t k0) {
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + a_r + 16 * i, k = k0 + a_k;
        ra[i] = (row < M && k < K) ? *(const float4*)(A + row * g.lda + k) : make_float4(0, 0, 0, 0);
        const int64_t kb = k0 + b_r + 16 * i;
        rb[i] = (b_nvalid && kb < K) ? *(const float4*)(B + kb * g.ldb + b_col) : make_float4(0, 0, 0, 0);
      }
    };
    gload(0);
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        As[a_r + 16 * i][a_k + 0] = ra[i].x;
        As[a_r + 16 * i][a_k + 1] = ra[i].y;
        As[a_r + 16 * i][a_k + 2] = ra[i].z;
        As[a_r + 16 * i][a_k + 3] = ra[i].w;
        *(float4*)&Bs[b_r + 16 * i][b_n] = rb[i];
      }
      __syncthreads();
      if (k0 + TK < K) gload(k0 + TK);
  #pragma unroll
      for (int kk = 0; kk < TK; kk += 4) {
        float a[2], b[2];
  #pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[wm * 32 + i * 16 + (lane & 15)][kk + (lane >> 4)];
  #pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bs[kk + (lane >> 4)][wn * 32 + j * 16 + (lane & 15)];
  #pragma unroll
        for (int i = 0; i < 2; ++i)
  #pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }

  #pragma unroll
    for (int i = 0; i < 2; ++i)
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (col >= N) continue;
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
          if (row >= M) continue;
          float v = acc[i][j][r];
          if (EPI == EPI_GELU_TANH) v = gelu_tanh_f32(v);
          float* c = (float*)g.C + row * g.ldc + col;
          if (EPI == EPI_ACC_F32) v = *c + v;
          *c = v;
        }
      }
  }  // tile loop
}

}  // namespace

hipError_t launch_gemm_f32(const GemmDesc& g, hipStream_t stream) {
  const int64_t tm = (g.M + TM - 1) / TM, tn = (g.N + TN - 1) / TN;
  if (tm <= 0 || tn <= 0) return hipSuccess;
  // one workgroup per tile up to 2^20 of them; beyond that the workgroups loop over the tiles
  const int64_t tiles = tm * tn;
  dim3 grid((unsigned)(tiles < ((int64_t)1 << 20) ? tiles : ((int64_t)1 << 20))), block(NT);
  switch (g.epi) {
    case EPI_STORE:
    case EPI_PARTIAL_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, block, 0, stream, g); break;
    case EPI_GELU_TANH: hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU_TANH>, grid, block, 0, stream, g); break;
    case EPI_ACC_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_ACC_F32>, grid, block, 0, stream, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
