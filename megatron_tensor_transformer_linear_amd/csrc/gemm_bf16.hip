// bf16 GEMM launcher: the LAY_NN kernels (forward products X.W) and the dispatch over
// operand layouts (the launch planner is in gemm_plan.hip).  The kernel itself is in gemm_bf16_kernel.hpp; the LAY_NT
// and LAY_TN kernels of the backward products are built in gemm_bf16_nt.hip and
// gemm_bf16_tn.hip.
#include "gemm_bf16_kernel.hpp"

namespace tpk {

hipError_t launch_shape_nn(int bm, int bn, const GemmDesc& g, hipStream_t stream) {
  return launch_shape_t<LAY_NN>(bm, bn, g, stream);
}

namespace {
hipError_t launch_shape(int bm, int bn, const GemmDesc& g, hipStream_t stream) {
  switch (g.layout) {
    case LAY_NN: return launch_shape_nn(bm, bn, g, stream);
    case LAY_NT: return launch_shape_nt(bm, bn, g, stream);
    case LAY_TN: return launch_shape_tn(bm, bn, g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_plan(const GemmPlan& pl, const GemmDesc& g, hipStream_t stream) {
  GemmDesc a = g;
  a.N = pl.n0;
  hipError_t e = launch_shape(pl.bm0, pl.bn0, a, stream);
  if (e != hipSuccess || pl.n1 == 0) return e;
  GemmDesc b = g;
  b.N = pl.n1;
  b.n_off = g.n_off + pl.n0;
  const size_t es = g.epi == EPI_PARTIAL_F32 || g.epi == EPI_ACC_F32 ? 4 : 2;
  b.C = (char*)g.C + (size_t)pl.n0 * es;
  if (g.aux) b.aux = (char*)g.aux + (size_t)pl.n0 * 2;
  return launch_shape(pl.bm1, pl.bn1, b, stream);
}
}  // namespace

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t stream) {
  return launch_plan(gemm_bf16_plan(g.M, g.N, device_cus()), g, stream);
}

// Split of the narrow strip's contraction.  The strip of a plan is the columns that do not
// fill a whole round of 256 x 256 tiles; as 128 x 128 tiles it runs at half the rate of the
// wide part (each 128 x 128 tile does a quarter of the MFMA work per K step for half the
// loads).  Computed instead as 256 x 256 tiles over GEMM_KSPLIT contraction ranges, the
// strip's tiles times GEMM_KSPLIT fill the compute units (the 8192 x 512 strip of the block's
// QKV projection: 64 tiles x 4 = 256 work items), and the reduce kernel sums the fp32
// partials in split order into the bf16 output.
hipError_t launch_gemm_bf16_split(const GemmDesc& g, float* ws, hipStream_t stream) {
  const GemmPlan pl = gemm_bf16_plan(g.M, g.N, device_cus());
  if (!ws || !gemm_split_applies(pl, g.K) || g.epi != EPI_STORE || g.layout != LAY_NN)
    return launch_plan(pl, g, stream);
  GemmDesc a = g;
  a.N = pl.n0;
  hipError_t e = launch_shape(pl.bm0, pl.bn0, a, stream);
  if (e != hipSuccess) return e;
  GemmDesc b = g;  // the strip: GEMM_KSPLIT fp32 partials [M, n1], dense, one after another
  b.N = pl.n1;
  b.n_off = g.n_off + pl.n0;
  b.C = ws;
  b.ldc = pl.n1;
  b.epi = EPI_PARTIAL_F32;
  b.ksplit = GEMM_KSPLIT;
  b.c_split_stride = g.M * pl.n1;
  e = launch_shape(256, 256, b, stream);
  if (e != hipSuccess) return e;
  ReduceDesc r;
  r.parts = ws;
  r.n_parts = GEMM_KSPLIT;
  r.part_stride = g.M * pl.n1;
  r.residual = nullptr;
  r.gamma = nullptr;
  r.beta = nullptr;
  r.eps = 0.0f;
  r.h_out = (bf16_t*)g.C + pl.n0;
  r.y_out = nullptr;
  r.rows = g.M;
  r.H = pl.n1;
  r.bf16 = 1;
  r.ld_out = g.ldc;
  return launch_reduce_ln(r, stream);
}

}  // namespace tpk
