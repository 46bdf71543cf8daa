// bf16 GEMM launcher: the LAY_NN kernels (forward products X.W), the launch planner and the
// dispatch over operand layouts.  The kernel itself is in gemm_bf16_kernel.hpp; the LAY_NT
// and LAY_TN kernels of the backward products are built in gemm_bf16_nt.hip and
// gemm_bf16_tn.hip.
#include <atomic>

#include "gemm_bf16_kernel.hpp"

namespace tpk {

// The count is cached per device in atomics: concurrent first calls on one device may both
// query it, and both store the same value.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_shape_nn(int bm, int bn, const GemmDesc& g, hipStream_t stream) {
  return launch_shape_t<LAY_NN>(bm, bn, g, stream);
}

// Launch plan for one product: the tile shapes and, optionally, a split of the N range into a
// part of 256 x 256 tiles that fills whole rounds of workgroups and a strip of 128 x 128
// tiles.  The plan minimises the sum over launches of rounds x the measured cost of one round
// of that tile shape relative to a round of 256 x 256 tiles (MI355X, K = 12288, per-round
// time ratios 256x192 0.862, 256x128 0.693, 128x128 0.455).  For the 8192 x 4608 QKV
// projection that is 4096 columns of 256 x 256 tiles (two rounds) plus a 512-wide strip of
// 128 x 128 tiles (one round): 726 us against 792 us for 256 x 192 tiles alone.
GemmPlan gemm_bf16_plan(int64_t M, int64_t N, int cus) {
  struct Shape {
    int bm, bn;
    double cost;
  };
  const Shape shapes[] = {{256, 256, 1.0}, {256, 192, 0.862}, {256, 128, 0.693}, {128, 128, 0.455}};
  auto rounds = [&](const Shape& sh, int64_t n) {
    const int64_t tiles = ((M + sh.bm - 1) / sh.bm) * ((n + sh.bn - 1) / sh.bn);
    return (tiles + cus - 1) / cus;
  };
  GemmPlan best{256, 256, N, 0, 0, 0};
  double best_cost = -1.0;
  for (const Shape& sh : shapes) {
    const double c = rounds(sh, N) * sh.cost;
    if (best_cost < 0 || c < best_cost - 1e-9) {
      best = GemmPlan{sh.bm, sh.bn, N, 0, 0, 0};
      best_cost = c;
    }
  }
  // Split: the widest multiple of 256 columns whose 256 x 256 tiles fill whole rounds.
  const int64_t tm = (M + 255) / 256;
  for (int64_t nm = (N / 256) * 256; nm >= 256; nm -= 256) {
    if ((tm * (nm / 256)) % cus != 0) continue;
    if (nm == N) break;
    const double c = rounds(shapes[0], nm) * shapes[0].cost + rounds(shapes[3], N - nm) * shapes[3].cost;
    if (c < best_cost - 1e-9) {
      best = GemmPlan{256, 256, nm, 128, 128, N - nm};
      best_cost = c;
    }
    break;
  }
  return best;
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
// loads).  Computed instead as 256 x 256 tiles over KSPLIT contraction ranges, the strip's
// tiles times KSPLIT fill the compute units (the 8192 x 512 strip of the block's QKV
// projection: 64 tiles x 4 = 256 work items), and the reduce kernel sums the fp32 partials
// in split order into the bf16 output.
namespace {
constexpr int KSPLIT = 4;

bool split_applies(const GemmPlan& pl, int64_t K) {
  return pl.n1 > 0 && pl.bm1 == 128 && K % (KSPLIT * 8) == 0;
}
}  // namespace

int64_t gemm_bf16_split_workspace(int64_t M, int64_t N, int64_t K) {
  const GemmPlan pl = gemm_bf16_plan(M, N, device_cus());
  return split_applies(pl, K) ? (int64_t)KSPLIT * M * pl.n1 * 4 : 0;
}

hipError_t launch_gemm_bf16_split(const GemmDesc& g, float* ws, hipStream_t stream) {
  const GemmPlan pl = gemm_bf16_plan(g.M, g.N, device_cus());
  if (!ws || !split_applies(pl, g.K) || g.epi != EPI_STORE || g.layout != LAY_NN)
    return launch_plan(pl, g, stream);
  GemmDesc a = g;
  a.N = pl.n0;
  hipError_t e = launch_shape(pl.bm0, pl.bn0, a, stream);
  if (e != hipSuccess) return e;
  GemmDesc b = g;  // the strip: KSPLIT fp32 partials [M, n1], dense, one after another
  b.N = pl.n1;
  b.n_off = g.n_off + pl.n0;
  b.C = ws;
  b.ldc = pl.n1;
  b.epi = EPI_PARTIAL_F32;
  b.ksplit = KSPLIT;
  b.c_split_stride = g.M * pl.n1;
  e = launch_shape(256, 256, b, stream);
  if (e != hipSuccess) return e;
  ReduceDesc r;
  r.parts = ws;
  r.n_parts = KSPLIT;
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
