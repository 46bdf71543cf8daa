// bf16 MFMA GEMM tile for gfx950 with the column / row-parallel epilogues.
//
//   C[M, N] = epi( A[M, K] . B[K, N] ),  A and B bf16 row-major, fp32 accumulation.
//
// Used for the column-parallel linear (epilogue: optional GeLU-tanh, bf16 store at the
// rank's column block), the row-parallel partial (epilogue: dense fp32 store) and the QKV /
// O projections of the attention-head shard (0539edu.com TP tutorial section 1.1, formula
// 1.1 and figure 1.2: the two block views of a matrix product that make the column and
// outer-product-sum splits).
//
// Tile: 256 x 256 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave owning a 128 x 128
// sub-tile as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).
// Operands are staged HBM -> registers -> LDS, double-buffered, one barrier per K step:
//   - A tile [256][64] is K-contiguous, as the MFMA A operand wants (8 consecutive k per
//     lane): one 16-byte LDS read per fragment.  Row pitch 72 elements keeps the 8 lanes of
//     each 16-byte LDS phase on distinct banks.
//   - B tile [64][256] keeps W's row-major layout (N-contiguous).  The MFMA B operand needs
//     8 consecutive k per lane; the gfx950 LDS transpose read ds_read_b64_tr_b16 delivers
//     exactly that: within each 16-lane group, lane 4q+c receives element c of the 8-byte
//     rows addressed by lanes q, q+4, q+8, q+12.  Pointing lane (q + 4s) at row k0+s,
//     columns n0+4q..4q+3 leaves lane i holding column n0+i, rows k0..k0+3; two reads give
//     the 8 k values.  Row pitch 272 elements puts the 4 rows of a read on distinct banks.
// Block -> tile mapping is XCD-aware: workgroups are dispatched round-robin over the 8 XCDs,
// so consecutive logical tiles are given to the same XCD (shared L2), and logical tiles
// walk 8-tile-row groups so an XCD's tiles share A and B panels.
#include "common.hpp"

namespace tpk {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHREADS = 256;
constexpr int A_PITCH = BK + 8;   // elements (144 B)
constexpr int B_PITCH = BN + 16;  // elements (544 B)
constexpr int A_STAGE = BM * A_PITCH;
constexpr int B_STAGE = BK * B_PITCH;
constexpr int SMEM_ELEMS = 2 * A_STAGE + 2 * B_STAGE;  // 143360 bytes

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;

__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const bf16_t* p, int second_offset) {
  const lds_bf16_t* lp = (const lds_bf16_t*)p;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lp);
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lp + second_offset));
  i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ void tile_coords(int bid, int tm, int tn, int& tile_m, int& tile_n) {
  const int nt = tm * tn;
  const int full = nt & ~7;
  int L = bid;
  if (bid < full) L = (bid & 7) * (full >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int per_group = G * tn;
  const int grp = L / per_group;
  const int first_m = grp * G;
  const int gsz = min(G, tm - first_m);
  const int w = L - grp * per_group;
  tile_m = first_m + w % gsz;
  tile_n = w / gsz;
}

template <int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmDesc g) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[SMEM_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t M = g.M, N = g.N, K = g.K;
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  int tile_m, tile_n;
  tile_coords(blockIdx.x, tm, tn, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  const bf16_t* __restrict__ A = (const bf16_t*)g.A;
  const bf16_t* __restrict__ B = (const bf16_t*)g.B;
  const int64_t lda = g.lda, ldb = g.ldb;

  // Per-thread global coordinates of the staged chunks (16 bytes = 8 elements each).
  const int a_row = tid >> 3, a_kc = (tid & 7) * 8;     // rows a_row + 32 i
  const int b_row = tid >> 5, b_nc = (tid & 31) * 8;    // k-rows b_row + 8 i
  const int64_t b_nlog = n0 + b_nc;
  const bool b_nvalid = b_nlog < N;
  const int64_t b_col = (b_nlog / g.b_blk) * g.b_blk_stride + (b_nlog % g.b_blk);

  // Staging loads are raw buffer loads: the hardware returns zeros for any offset past the
  // resource's byte range, so tile edges need neither branches nor selects.  A's resource
  // covers the tile's rows (rows >= M fall outside it); B's resource is re-based at every K
  // step and covers the remaining K rows of that step.  Chunks past K (for A) or past N (for
  // B) are given an offset outside every range.
  constexpr uint32_t OOB = 0x80000000u;
  const int64_t a_rows = min((int64_t)BM, M - m0);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + m0 * lda), (short)0, (int)(a_rows * lda * 2), 0x00020000);
  uint32_t a_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a_off[i] = (uint32_t)(((a_row + 32 * i) * lda + a_kc) * 2);
  uint32_t b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b_off[i] = b_nvalid ? (uint32_t)(((b_row + 8 * i) * ldb + b_col) * 2) : OOB;

  uint4 ra[8], rb[8];
  auto gload = [&](int64_t k0) {
    const bool a_kok = k0 + a_kc < K;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rsrc_a, a_kok ? a_off[i] + (uint32_t)(k0 * 2) : OOB, 0, 0));
    const int64_t k_rows = min((int64_t)BK, K - k0);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + k0 * ldb), (short)0, (int)(k_rows * ldb * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, b_off[i], 0, 0));
  };
  auto sstore = [&](int buf) {
    bf16_t* as = smem + buf * A_STAGE;
    bf16_t* bs = smem + 2 * A_STAGE + buf * B_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(as + (a_row + 32 * i) * A_PITCH + a_kc) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(bs + (b_row + 8 * i) * B_PITCH + b_nc) = rb[i];
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Lane-constant parts of the LDS fragment addresses.
  const int a_frag_row = wm * 128 + (lane & 31);
  const int a_frag_k = 8 * (lane >> 5);
  const int grp = lane >> 4, li = lane & 15;
  const int b_frag_krow = 8 * (grp >> 1) + (li >> 2);
  const int b_frag_col = wn * 128 + 16 * (grp & 1) + 4 * (li & 3);

  // Fragments are double-buffered in registers: the LDS reads of sub-step ks+1 are issued
  // before the 16 MFMAs of sub-step ks, so their latency hides behind the matrix work.
  bf16x8_t fa[2][4], fb[2][4];
  auto load_frags = [&](const bf16_t* as, const bf16_t* bs, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[slot][i] = *(const bf16x8_t*)(as + (a_frag_row + 32 * i) * A_PITCH + ks * 16 + a_frag_k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[slot][j] = ds_read_tr_pair(bs + (ks * 16 + b_frag_krow) * B_PITCH + b_frag_col + 32 * j,
                                    4 * B_PITCH);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };

  const int nk = (int)((K + BK - 1) / BK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const bf16_t* as = smem + cur * A_STAGE;
    const bf16_t* bs = smem + 2 * A_STAGE + cur * B_STAGE;
    // The scheduling fences keep this order; without them the compiler sinks each fragment
    // read next to its first use and the LDS latency is exposed before every MFMA group.
    if (more) gload((int64_t)(kt + 1) * BK);
    load_frags(as, bs, 0, 0);
    load_frags(as, bs, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(as, bs, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(as, bs, 3, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) sstore(cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element r of block (i, j) sits at
  //   row = 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,  col = 32 j + lane % 32
  // of the wave's 128 x 128 sub-tile.
  const int64_t ldc = g.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        float v = acc[i][j][r];
        if (EPI == EPI_PARTIAL_F32) {
          ((float*)g.C)[row * ldc + col] = v;
        } else {
          if (EPI == EPI_GELU_TANH) v = gelu_tanh_f32(v);
          ((bf16_t*)g.C)[row * ldc + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t stream) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  const int64_t blocks = tm * tn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (g.epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE>, grid, block, 0, stream, g); break;
    case EPI_GELU_TANH: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_GELU_TANH>, grid, block, 0, stream, g); break;
    case EPI_PARTIAL_F32: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_PARTIAL_F32>, grid, block, 0, stream, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
