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
// Tile: 256 x BN x 32 per K step (BN = 256, 192 or 128), 256 threads = 4 waves in a 2 x 2
// grid, each wave owning a 128 x BN/2 sub-tile as 4 x (BN/64) blocks of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators in AGPRs).
//
// Staging: HBM -> LDS directly (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at
// LDS base + 16 * lane, no VGPR round trip), in a ring of 4 stages, so the loads of stage
// kt + 4 are issued while stage kt is being multiplied, three K steps ahead of their use.
// The data arrangement inside a stage is chosen by which global chunk each lane fetches:
//   - A stage [256 rows][32 k] (64 B per row, K-contiguous as the MFMA A operand wants):
//     row r keeps its four 16-byte k-chunks XOR-permuted by (r >> 2) & 3.  The LDS serves a
//     16-byte read 16 lanes at a time from 64 four-byte banks (measured with the bank-conflict
//     counter: 16 consecutive lanes over 256 contiguous bytes run conflict-free), and this
//     permutation gives the 16 rows of each such group distinct 16-byte bank groups.
//   - B stage [32 k-rows][256 columns] (N-contiguous, W's own layout): k-row k keeps its
//     16-byte column chunks XOR-permuted by 4 (k & 3) ^ 2 ((k >> 1) & 1), which puts the
//     4 rows x 32 bytes of each transpose read on distinct banks.
// The MFMA B operand needs 8 consecutive k per lane; the gfx950 LDS transpose read
// ds_read_b64_tr_b16 delivers them from the N-contiguous tile: within each 16-lane group,
// lane 4q+c receives element c of the 8-byte rows addressed by lanes q, q+4, q+8, q+12, so
// pointing lane (q + 4s) at k-row k0+s, columns n0+4q..4q+3 leaves lane i holding column
// n0+i, k-rows k0..k0+3; two reads give the 8 k values.
// Per K step each wave issues its fragment reads for the second half-step under the
// MFMAs of the first, waits for its own loads of the next stage, meets the other waves at
// one barrier, queues the next stage's loads into the buffer just drained, and reads the
// next stage's first fragments under the MFMAs of the second half-step.
// Block -> tile mapping is XCD-aware: workgroups are dispatched round-robin over the 8 XCDs,
// so consecutive logical tiles are given to the same XCD (shared L2), and logical tiles
// walk 8-tile-row groups so an XCD's tiles share A and B panels.
#include <type_traits>

#include "common.hpp"

namespace tpk {
namespace {

constexpr int BM = 256, BK = 32;
constexpr int NTHREADS = 256;
constexpr int A_BYTES = BM * BK * 2;  // one A stage: 16 KB
constexpr uint32_t OOB = 0x80000000u; // buffer offset past every resource range

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt[3:0] in
// bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// vmcnt(N) and lgkmcnt(0) together.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the release/acquire fences of __syncthreads (those would wait
// for every outstanding LDS-bound load); memory order is kept by the explicit waits.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Raw buffer resource: base address, no stride, `bytes` bytes in range (loads at offsets at
// or past it return zeros), raw-buffer flags.  The arguments are wave-uniform; the resource
// is made to live in scalar registers.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// One direct-to-LDS 16-byte load per lane: lane i's 16 bytes, read from buffer offset
// voff + soff, land at LDS address lds_base + IMM + 16 i.  Issued through inline assembly
// so that the compiler does not order LDS reads after it with a full vector-memory wait;
// completion is tracked by the explicit vmcnt waits of the K loop.  M0 (the LDS address of
// the load) is set here and used by nothing else in the kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <uint32_t IMM>
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, i32x4_t rsrc, uint32_t soff) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
               :: "s"(lds_base), "i"(IMM), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const char* p, int second_offset) {
  const lds_char_t* lp = (const lds_char_t*)p;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lp);
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lp + second_offset));
  i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ int swz_a(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz_b(int krow) { return (4 * (krow & 3)) ^ (2 * ((krow >> 1) & 1)); }

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

template <int BN, int NST, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmDesc g) {
  constexpr int WN = BN / 2;                      // columns per wave
  constexpr int NJ = WN / 32;                     // 32-wide MFMA blocks per wave
  constexpr int BPITCH = BN == 128 ? 256 : 512;   // bytes per B k-row in LDS
  constexpr int CPR = BPITCH / 16;                // 16-byte chunks per B k-row
  constexpr int RPI = 1024 / BPITCH;              // B k-rows per wave load instruction
  constexpr int B_BYTES = BK * BPITCH;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LD = A_BYTES / 1024 / 4;        // load instructions per wave per stage
  constexpr int B_LD = B_BYTES / 1024 / 4;
  constexpr int LPS = A_LD + B_LD;
  static_assert(BN == 256 || BN == 192 || BN == 128, "tile width");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;

  const int64_t M = g.M, N = g.N, K = g.K;
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  int tile_m, tile_n;
  tile_coords(blockIdx.x, tm, tn, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  const bf16_t* __restrict__ A = (const bf16_t*)g.A;
  const bf16_t* __restrict__ B = (const bf16_t*)g.B;
  const int64_t lda = g.lda, ldb = g.ldb;

  // ---- per-lane source offsets of the direct-to-LDS loads
  // A: instruction i of wave wv fills rows 16 (4 wv + i) .. +15 of the stage, 4 lanes a row.
  const int64_t a_rows = min((int64_t)BM, M - m0);
  const i32x4_t rsrc_a = buffer_rsrc(A + m0 * lda, a_rows * lda * 2);
  uint32_t a_off[A_LD];
  int a_k[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = 16 * (A_LD * wv + i) + (lane >> 2);
    const int c = (lane & 3) ^ swz_a(row);
    a_k[i] = 8 * c;
    a_off[i] = (uint32_t)((row * lda + 8 * c) * 2);
  }
  // B: instruction i of wave wv fills k-rows RPI (B_LD wv + i) .. of the stage.
  uint32_t b_off[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int krow = RPI * (B_LD * wv + i) + lane / CPR;
    const int j = (lane % CPR) ^ swz_b(krow);
    const int64_t nlog = n0 + 8 * j;
    const bool ok = 8 * j < BN && nlog < N;
    const int64_t col = (nlog / g.b_blk) * g.b_blk_stride + (nlog % g.b_blk);
    b_off[i] = ok ? (uint32_t)((krow * ldb + col) * 2) : OOB;
  }

  // ---- per-lane LDS fragment offsets (bytes within a stage)
  const int r32 = lane & 31, kh = lane >> 5;
  int a_rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    a_rd[ks] = (wm * 128 + r32) * 64 + (((2 * ks + kh) ^ swz_a(r32)) * 16);
  const int grp = lane >> 4, li = lane & 15, q = li & 3, s = li >> 2;
  int b_rd[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int chunk = (wn * WN) / 8 + 4 * j + 2 * (grp & 1) + (q >> 1);
    b_rd[j] = A_BYTES + (8 * (grp >> 1) + s) * BPITCH + ((chunk ^ swz_b(s)) * 16) + (q & 1) * 8;
  }

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  bf16x8_t fa[2][4], fb[2][NJ];

  const int nk = (int)((K + BK - 1) / BK);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t*)smem;
  const uint32_t lds_a = lds0 + (uint32_t)(wv * A_LD * 1024);            // this wave's A loads
  const uint32_t lds_b = lds0 + (uint32_t)(A_BYTES + wv * B_LD * 1024);  // this wave's B loads

  // ---- the work items a K step is made of
  constexpr int NM = 4 * NJ;  // MFMAs per half-step
  constexpr int NR = 4 + NJ;  // fragment-read items per half-step (a B item is two reads)
  // MFMA m of a half-step: row block m / NJ, column block m % NJ.
  auto mfma = [&](int slot, int m) {
    const int i = m / NJ, j = m % NJ;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };
  // Read item t of sub-step ks of the stage held in buffer `buf` into fragment slot `slot`.
  auto read_item = [&](int buf, int ks, int slot, int t) {
    const char* sb = smem + buf * STAGE;
    if (t < 4) {
      fa[slot][t] = *(const bf16x8_t*)(sb + a_rd[ks] + t * 32 * 64);
    } else {
      const int j = t - 4;
      fb[slot][j] = ds_read_tr_pair(sb + b_rd[j] + ks * 16 * BPITCH, 4 * BPITCH);
    }
  };
  // Load item U of stage kd into buffer BUF (U < A_LD: an A load, else a B load).  Parts of
  // the stage past K, and whole stages past K, come back as zeros (out-of-range offsets or
  // an empty B range), so the K loop can run whole groups of NST steps.  The B resource is
  // re-based at every stage so that its range check alone bounds the rows read.
  const int Ki = (int)K;                       // K < 2^31 (bounded by the leading dimensions)
  const int ldb2 = (int)(ldb * 2);             // bytes per B row
  const char* const Bbytes = (const char*)B;
  auto dma_item = [&](auto BUFC, auto UC, int kd) {
    constexpr int BUF = decltype(BUFC)::value, U = decltype(UC)::value;
    const int k0 = kd * BK;
    if constexpr (U < A_LD) {
      const uint32_t off = a_k[U] < Ki - k0 ? a_off[U] : OOB;
      dma16<BUF * STAGE + U * 1024>(lds_a, off, rsrc_a, (uint32_t)k0 * 2u);
    } else {
      constexpr int I = U - A_LD;
      const int k_rows = max(0, min(BK, Ki - k0));
      const i32x4_t rsrc_b = buffer_rsrc(Bbytes + (int64_t)k0 * ldb2, (int64_t)(k_rows * ldb2));
      dma16<BUF * STAGE + I * 1024>(lds_b, b_off[I], rsrc_b, 0u);
    }
  };

  // One K step on the stage in buffer S (kt % NST == S).  First half: the MFMAs of sub-step 0,
  // with the reads of sub-step 1 and the second half of stage kt+NST-1's loads (into buffer
  // S-1, free since the previous step's barrier) between them.  Then the wait for this
  // wave's loads of stage kt+1 (the NST-2 later stages may still be in flight) and the
  // barrier, after which every wave's share of stage kt+1 has landed and buffer S is no
  // longer read.  Second half: the MFMAs of sub-step 1, with the reads of stage kt+1's
  // sub-step 0 and the first half of stage kt+NST's loads (into buffer S) between them.
  // Splitting each stage's loads over two half-steps keeps the four waves' 1 KB loads from
  // arriving at the address unit in one burst.  Each item is fenced in place, so the issue
  // order is exactly this interleave.
  constexpr int LH = LPS / 2;  // loads of a stage issued in the second half of a step
  auto half_step = [&](auto SC, auto SLOTC, auto LOC, auto HIC, auto RBUFC, int ks_read,
                       int read_slot, auto DBUFC, int kd) {
    constexpr int SLOT = decltype(SLOTC)::value;
    constexpr int LO = decltype(LOC)::value, HI = decltype(HIC)::value;  // load items [LO, HI)
    constexpr int RBUF = decltype(RBUFC)::value;
    constexpr int NITEM = NR + (HI - LO);
    (void)SC;
    static_for<NM>([&](auto MC) {
      constexpr int m = decltype(MC)::value;
      mfma(SLOT, m);
      __builtin_amdgcn_sched_barrier(0);
      static_for<NITEM>([&](auto TC) {
        constexpr int t = decltype(TC)::value;
        if constexpr (t * NM / NITEM == m) {
          if constexpr (t < NR) read_item(RBUF, ks_read, read_slot, t);
          else dma_item(DBUFC, std::integral_constant<int, LO + t - NR>{}, kd);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto step = [&](auto SC, int kt) {
    constexpr int S = decltype(SC)::value;
    half_step(SC, std::integral_constant<int, 0>{}, std::integral_constant<int, LH>{},
              std::integral_constant<int, LPS>{}, SC, 1, 1,
              std::integral_constant<int, (S + NST - 1) % NST>{}, kt + NST - 1);
    wait_vmcnt_lgkm0<(NST - 2) * LPS>();
    lds_barrier();
    half_step(SC, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{},
              std::integral_constant<int, LH>{}, std::integral_constant<int, (S + 1) % NST>{}, 0, 0,
              SC, kt + NST);
  };

  // ---- prologue: stages 0 .. NST-2 in flight, the first half of stage NST-1 (its second
  // half goes out in the first step), stage 0 landed, its first fragments read
  static_for<NST - 1>([&](auto SC) {
    static_for<LPS>([&](auto UC) { dma_item(SC, UC, decltype(SC)::value); });
  });
  static_for<LH>([&](auto UC) {
    dma_item(std::integral_constant<int, NST - 1>{}, UC, NST - 1);
  });
  wait_vmcnt<(NST - 2) * LPS + LH>();
  lds_barrier();
#pragma unroll
  for (int t = 0; t < NR; ++t) read_item(0, 0, 0, t);

  // ---- main loop over groups of NST steps (the last group may run on zero-filled stages)
  const int ngroups = (nk + NST - 1) / NST;
  for (int gi = 0; gi < ngroups; ++gi) {
    const int kt = gi * NST;
    static_for<NST>([&](auto SC) { step(SC, kt + decltype(SC)::value); });
  }
  // Loads of the stages past the end are still in flight: let them land before the LDS is
  // reused or released.
  wait_vmcnt<0>();

  // Epilogue.  Accumulator element r of block (i, j) sits at
  //   row = 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,  col = 32 j + lane % 32
  // of the wave's 128 x WN sub-tile.
  const int64_t ldc = g.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = n0 + wn * WN + 32 * j + (lane & 31);
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

template <int BN, int NST>
hipError_t launch_bn(const GemmDesc& g, hipStream_t stream) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  const int64_t blocks = tm * tn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (g.epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_kernel<BN, NST, EPI_STORE>), grid, block, 0, stream, g); break;
    case EPI_GELU_TANH: hipLaunchKernelGGL((gemm_bf16_kernel<BN, NST, EPI_GELU_TANH>), grid, block, 0, stream, g); break;
    case EPI_PARTIAL_F32: hipLaunchKernelGGL((gemm_bf16_kernel<BN, NST, EPI_PARTIAL_F32>), grid, block, 0, stream, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Tile width per shape: the fewest rounds of workgroups over the 256 compute units, each
// round costing its tile width, ties going to the wider tile.
int gemm_bf16_tile_n(int64_t M, int64_t N) {
  const int64_t tm = (M + BM - 1) / BM;
  int best = 256;
  int64_t best_cost = -1;
  for (int bn : {256, 192, 128}) {
    const int64_t tiles = tm * ((N + bn - 1) / bn);
    const int64_t cost = ((tiles + 255) / 256) * bn;
    if (best_cost < 0 || cost < best_cost) { best = bn; best_cost = cost; }
  }
  return best;
}

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t stream) {
  switch (gemm_bf16_tile_n(g.M, g.N)) {
    case 192: return launch_bn<192, 4>(g, stream);
    case 128: return launch_bn<128, 4>(g, stream);
    default: return launch_bn<256, 4>(g, stream);
  }
}

}  // namespace tpk
