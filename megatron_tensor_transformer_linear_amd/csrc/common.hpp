// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Epilogues of the GEMM tile.
enum Epilogue : int {
  EPI_STORE = 0,        // Y (io dtype) = acc
  EPI_GELU_TANH = 1,    // Y (io dtype) = gelu_tanh(acc)
  EPI_PARTIAL_F32 = 2,  // Z (fp32) = acc
  EPI_GELU_SAVE = 3,    // Y (bf16) = gelu_tanh(acc), and aux (bf16) = acc, the pre-activation
  EPI_GELU_BWD = 4,     // Y (bf16) = acc * gelu_tanh'(aux), aux the bf16 pre-activation
  EPI_ACC_F32 = 5       // Z (fp32) += acc
};

// Memory layouts of the two GEMM operands (bf16 tile only).  Bit 0: A is stored
// M-contiguous (the product reads X^T of a row-major X).  Bit 1: B is stored K-contiguous
// (the product reads W^T of a row-major W).
enum Layout : int {
  LAY_NN = 0,  // A [M, K] and B [K, N] row-major
  LAY_TN = 1,  // A^T [K, M] row-major (element (m, k) at A + k lda + m), B [K, N] row-major
  LAY_NT = 2   // A [M, K] row-major, B^T [N, K] row-major (element (k, n) at B + n ldb + k)
};

// C = epi(A . B) for one rank's shard.
//   A [M, K] row-major, leading dimension lda, already offset to the rank's first column.
//   B [K, *] row-major, leading dimension ldb, already offset to the rank's first row and
//     first column.  Logical column n of B lives at physical column
//       (n / b_blk) * b_blk_stride + (n % b_blk)
//     which lets the QKV projection read three separated column blocks of [Wq | Wk | Wv]
//     as one operand (b_blk = N gives the plain contiguous case).
//     n_off shifts that logical numbering: column n of this product is logical column
//     n_off + n of B (0 unless the launcher splits N over several launches).
//   C [M, N] row-major, leading dimension ldc (bf16 / fp32 per dtype and epilogue).
//   layout: a Layout.  With LAY_NT the logical-to-physical column map of B must be the
//     identity (b_blk >= n_off + N); row n_off + n of B^T is column n.  With LAY_TN, A is
//     A^T [K, M] with leading dimension lda.
//   aux [M, N] bf16, leading dimension ldaux: the pre-activation written by EPI_GELU_SAVE
//     or read by EPI_GELU_BWD (unused otherwise).
struct GemmDesc {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int64_t b_blk;
  int64_t b_blk_stride;
  int64_t n_off;
  void* C;
  int64_t ldc;
  int64_t M, N, K;
  int epi;
  int layout = LAY_NN;
  void* aux = nullptr;
  int64_t ldaux = 0;
  // Split of the contraction (EPI_PARTIAL_F32 in LAY_NN only): work item s of a tile
  // contracts k in [s K / ksplit, (s + 1) K / ksplit) and writes its fp32 partial at
  // C + s * c_split_stride.  K / ksplit must be a multiple of 8.
  int ksplit = 1;
  int64_t c_split_stride = 0;
};

// Causal / full attention over one rank's heads.
//   qkv [batch*seq, 3*hl*d] bf16 = [Q_r | K_r | V_r], head h at columns h*d of each block.
//   out [batch*seq, hl*d] bf16, heads concatenated in ascending order.
struct AttnDesc {
  const bf16_t* qkv;
  bf16_t* out;
  int64_t batch, seq;
  int hl, d;
  int causal;
  float scale_log2;  // log2(e) / sqrt(d)
};

// h = residual + sum_p parts[p]; y = LayerNorm(h) * gamma + beta.
struct ReduceDesc {
  const float* parts;  // fp32 partials, or bf16 ones (parts_bf16) at the same address
  int n_parts;
  int64_t part_stride;
  const void* residual;
  const void* gamma;
  const void* beta;
  float eps;
  void* h_out;
  void* y_out;
  int64_t rows, H;
  int bf16;  // io dtype is bf16 (else fp32)
  int64_t ld_out = 0;  // row pitch of h_out and y_out in elements (0: H)
  int parts_bf16 = 0;  // the partials are bf16 (bf16 io only)
};

// Tile shapes of one bf16 product: columns [0, n0) with bm0 x bn0 tiles, then, if n1 > 0,
// columns [n0, n0 + n1) with bm1 x bn1 tiles in a second launch.
struct GemmPlan {
  int bm0, bn0;
  int64_t n0;
  int bm1, bn1;
  int64_t n1;
};
GemmPlan gemm_bf16_plan(int64_t M, int64_t N, int cus);
// Contraction ranges of the narrow strip in launch_gemm_bf16_split, and whether a plan's strip
// is split that way (a strip of 128 x 128 tiles, K divisible into GEMM_KSPLIT ranges of whole
// 8-element chunks).
constexpr int GEMM_KSPLIT = 4;
inline bool gemm_split_applies(const GemmPlan& pl, int64_t K) {
  return pl.n1 > 0 && pl.bm1 == 128 && K % (GEMM_KSPLIT * 8) == 0;
}

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t stream);
// Compute units of the current device (cached per device; 256 when it cannot be queried).
int device_cus();
// Workspace bytes launch_gemm_bf16_split needs for an M x N product: the fp32 partials of the
// narrow strip of the launch plan (0 when the plan has no strip).
int64_t gemm_bf16_split_workspace(int64_t M, int64_t N, int64_t K);
// launch_gemm_bf16 for a plain bf16 store (EPI_STORE, LAY_NN), with the plan's narrow strip
// computed as 256 x 256 tiles over KSPLIT contraction ranges into `ws` and summed into C by the
// reduce kernel; without a strip (or when K does not split) it is launch_gemm_bf16.
hipError_t launch_gemm_bf16_split(const GemmDesc& g, float* ws, hipStream_t stream);
hipError_t launch_gemm_f32(const GemmDesc& g, hipStream_t stream);
hipError_t launch_attention(const AttnDesc& a, hipStream_t stream);
hipError_t launch_reduce_ln(const ReduceDesc& r, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even: the gfx950 conversion instruction
// v_cvt_pk_bf16_f32 (checked on MI355X to give the same bits as the integer
// round-to-nearest-even formula on 16.7M finite values, including exact ties, both
// neighbours of a tie, denormals and values that round to infinity).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// GeLU, tanh form.  0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), so
//   gelu(x) = x / (1 + exp(-2u)),  u = sqrt(2/pi) (x + 0.044715 x^3),
// with exp evaluated as exp2 on the hardware transcendental unit.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float m2log2e = -2.0f * 1.4426950408889634f;
  float u = k0 * (x + k1 * x * x * x);
  float e = __builtin_amdgcn_exp2f(m2log2e * u);
  return x / (1.0f + e);
}

}  // namespace tpk
