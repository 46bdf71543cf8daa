// Host-side planning of the bf16 products: the compute-unit count, the tile shapes of a
// launch (gemm_bf16_plan) and the workspace of the split strip.  No device code.
#include <atomic>

#include "common.hpp"

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

int64_t gemm_bf16_split_workspace(int64_t M, int64_t N, int64_t K) {
  const GemmPlan pl = gemm_bf16_plan(M, N, device_cus());
  return gemm_split_applies(pl, K) ? (int64_t)GEMM_KSPLIT * M * pl.n1 * 4 : 0;
}

}  // namespace tpk
