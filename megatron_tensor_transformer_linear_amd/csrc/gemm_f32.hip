// fp32 MFMA GEMM tile for gfx950 (io dtype fp32): the column / row-parallel linears of the
// small fp32 MLP.  Same contract and epilogues as the bf16 tile (0539edu.com TP tutorial
// section 1.1, formula 1.1 and figure 1.2), built on v_mfma_f32_16x16x4_f32.
//
// Tile 64 x 64 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave 32 x 32 as 2 x 2 blocks
// of 16 x 16.  Operand layout of the 16x16x4 instruction: A lane l holds A[l % 16][l / 16],
// B lane l holds B[l / 16][l % 16]; accumulator element r of lane l is C[4 (l / 16) + r][l % 16].
// Each K step's global loads go out before the previous step is multiplied (held in
// registers), and the K step is 64 wide.
//
// Small products (fewer 64 x 64 tiles than a quarter of the compute units, as in the fp32 MLP
// of a few MFLOP) are latency-bound on that tile: a handful of workgroups each walk the whole
// contraction one K step after another (the row product of X[64, 512] . W[512, 256] is 4
// workgroups of 8 steps).  They use gemm_f32_small_kernel instead: 16 x 16 output tiles, 16
// times as many workgroups, the contraction split over the 4 waves of a workgroup, and the 4
// partial tiles summed through LDS in wave order (a fixed order: results are deterministic).
#include "common.hpp"

namespace tpk {
namespace {

constexpr int TM = 64, TN = 64, TK = 64;
constexpr int NT = 256;
constexpr int SK = 64;  // small kernel: k per wave in each block of 4 * SK

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

// Small products: one 16 x 16 output tile per workgroup.  Wave w contracts k in
// [kb + SK w, kb + SK (w + 1)) of every block kb of 4 SK, as 16 instructions of 4 k each; the
// four k of instruction (t, j) for lane group q = lane / 16 are kb + SK w + 16 t + 4 q + j, so
// that lane's A operands for t = 0..3 are one 16-byte load of 4 consecutive k of its row, and
// its B operands 4 loads of its column (16 consecutive columns per lane group: coalesced).
// The next block's loads are in flight while a block is multiplied.  K, lda and ldb are
// multiples of 8 and the operands 16-byte aligned (checked by the callers), so a 16-byte A load
// lies wholly inside or wholly past K.
template <int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_small_kernel(GemmDesc g) {
  __shared__ float red[4][64][4];  // each wave's partial tile, in accumulator order

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t M = g.M, N = g.N, K = g.K;
  const float* __restrict__ A = (const float*)g.A;
  const float* __restrict__ B = (const float*)g.B;
  const int64_t tn = (N + 15) / 16, ntiles = ((M + 15) / 16) * tn;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t m0 = (tile / tn) * 16, n0 = (tile % tn) * 16;
    const int64_t arow = m0 + r16, ncol = n0 + r16;
    const bool aok = arow < M, bok = ncol < N;
    const int64_t bcol = (ncol / g.b_blk) * g.b_blk_stride + (ncol % g.b_blk);

    float4 a[2][4];
    float b[2][4][4];
    auto load = [&](int64_t kb, int buf) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t k = kb + SK * w + 16 * t + 4 * q;
        const bool kin = k < K;
        a[buf][t] = aok && kin ? *(const float4*)(A + arow * g.lda + k) : make_float4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[buf][t][j] = bok && kin ? B[(k + j) * g.ldb + bcol] : 0.0f;
      }
    };
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto mult = [&](int buf) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float av[4] = {a[buf][t].x, a[buf][t].y, a[buf][t].z, a[buf][t].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], b[buf][t][j], acc, 0, 0, 0);
      }
    };
    load(0, 0);
    int64_t kb = 0;
    for (; kb + 8 * SK < K + 4 * SK; kb += 8 * SK) {  // two blocks per pass: buffers 0, 1
      load(kb + 4 * SK, 1);
      mult(0);
      if (kb + 8 * SK < K) load(kb + 8 * SK, 0);
      mult(1);
    }
    if (kb < K) mult(0);

#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][lane][r] = acc[r];
    __syncthreads();
    // thread tid: element (i, j) = (tid / 16, tid % 16), lane 16 (i / 4) + j, component i % 4
    const int i = tid >> 4, j = tid & 15;
    const int sl = 16 * (i >> 2) + j, sr = i & 3;
    float v = red[0][sl][sr] + red[1][sl][sr];
    v = v + red[2][sl][sr];
    v = v + red[3][sl][sr];
    const int64_t row = m0 + i, col = n0 + j;
    if (row < M && col < N) {
      if (EPI == EPI_GELU_TANH) v = gelu_tanh_f32(v);
      float* c = (float*)g.C + row * g.ldc + col;
      if (EPI == EPI_ACC_F32) v = *c + v;
      *c = v;
    }
    __syncthreads();  // red is rewritten by the next tile
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmDesc& g, hipStream_t stream) {
  const int64_t tm = (g.M + TM - 1) / TM, tn = (g.N + TN - 1) / TN;
  if (tm <= 0 || tn <= 0) return hipSuccess;
  const int64_t tiles = tm * tn;
  const int epi = g.epi == EPI_PARTIAL_F32 ? EPI_STORE : g.epi;
  if (epi != EPI_STORE && epi != EPI_GELU_TANH && epi != EPI_ACC_F32) return hipErrorInvalidValue;
  // one workgroup per tile up to 2^20 of them; beyond that the workgroups loop over the tiles
  const int64_t cap = (int64_t)1 << 20;
  if (tiles * 4 < device_cus()) {
    const int64_t st = ((g.M + 15) / 16) * ((g.N + 15) / 16);
    const dim3 grid((unsigned)(st < cap ? st : cap)), block(NT);
    if (epi == EPI_STORE) hipLaunchKernelGGL(gemm_f32_small_kernel<EPI_STORE>, grid, block, 0, stream, g);
    else if (epi == EPI_GELU_TANH) hipLaunchKernelGGL(gemm_f32_small_kernel<EPI_GELU_TANH>, grid, block, 0, stream, g);
    else hipLaunchKernelGGL(gemm_f32_small_kernel<EPI_ACC_F32>, grid, block, 0, stream, g);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(tiles < cap ? tiles : cap)), block(NT);
  if (epi == EPI_STORE) hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, block, 0, stream, g);
  else if (epi == EPI_GELU_TANH) hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU_TANH>, grid, block, 0, stream, g);
  else hipLaunchKernelGGL(gemm_f32_kernel<EPI_ACC_F32>, grid, block, 0, stream, g);
  return hipGetLastError();
}

}  // namespace tpk
