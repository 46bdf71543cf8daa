// bf16 MFMA GEMM tile for gfx950 with the column / row-parallel epilogues and their
// backward counterparts.
//
//   C[M, N] = epi( A[M, K] . B[K, N] ),  A and B bf16, fp32 accumulation.
//
// Used for the column-parallel linear (epilogue: optional GeLU-tanh, bf16 store at the
// rank's column block), the row-parallel partial (epilogue: dense fp32 store) and the QKV /
// O projections of the attention-head shard (0539edu.com TP tutorial section 1.1, formula
// 1.1 and figure 1.2: the two block views of a matrix product that make the column and
// outer-product-sum splits); in the backward pass, for the products with a transposed
// operand: dY = dZ . W^T (B read K-contiguous) and dW = X^T . dY (A read M-contiguous).
//
// Tile: BM x BN x 32 per K step (256 x 256, 256 x 192, 256 x 128 or 128 x 128, chosen per
// shape by gemm_bf16_plan), 256 threads = 4 waves in a 2 x 2 grid, each wave owning a
// BM/2 x BN/2 sub-tile as (BM/64) x (BN/64) blocks of v_mfma_f32_32x32x16_bf16 (fp32
// accumulators in AGPRs).
//
// Staging: HBM -> LDS directly (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at
// LDS base + 16 * lane, no VGPR round trip), in a ring of 4 stages, so the loads of stage
// kt + 4 are issued while stage kt is being multiplied, three K steps ahead of their use.
// Each operand's share of a stage takes one of two arrangements, set by how the operand is
// stored; which global chunk each lane fetches decides the arrangement:
//   - K-contiguous (A of X.W, or B read as W^T): [R rows][32 k], 64 B per row, the form the
//     MFMA operands take directly (one 16-byte read per lane).  Row r keeps its four 16-byte
//     k-chunks XOR-permuted by (r >> 2) & 3.  The LDS serves a 16-byte read 16 lanes at a
//     time from 64 four-byte banks (measured with the bank-conflict counter: 16 consecutive
//     lanes over 256 contiguous bytes run conflict-free), and this permutation gives the 16
//     rows of each such group distinct 16-byte bank groups.
//   - M- or N-contiguous (B as W is stored, or A read as X^T): [32 k-rows][R], k-row k
//     keeping its 16-byte chunks XOR-permuted by 4 (k & 3) ^ 2 ((k >> 1) & 1), which puts
//     the 4 rows x 32 bytes of each transpose read on distinct banks.  An MFMA operand needs
//     8 consecutive k per lane; the gfx950 LDS transpose read ds_read_b64_tr_b16 delivers
//     them: within each 16-lane group, lane 4q+c receives element c of the 8-byte rows
//     addressed by lanes q, q+4, q+8, q+12, so pointing lane (q + 4s) at k-row k0+s,
//     columns n0+4q..4q+3 leaves lane i holding column n0+i, k-rows k0..k0+3; two reads
//     give the 8 k values.  The A and B operands of the MFMA have the same lane layout
//     (lane l: row or column l % 32, k = 8 (l / 32) .. +7), so either arrangement serves
//     either operand.
// Per K step each wave issues its fragment reads for the second half-step under the
// MFMAs of the first, waits for its own loads of the next stage, meets the other waves at
// one barrier, queues the next stage's loads into the buffer just drained, and reads the
// next stage's first fragments under the MFMAs of the second half-step.
// Block -> tile mapping is XCD-aware: workgroups are dispatched round-robin over the 8 XCDs,
// so consecutive logical tiles are given to the same XCD (shared L2), and logical tiles
// walk 8-tile-row groups so an XCD's tiles share A and B panels.
//
// Each translation unit that includes this header instantiates the kernels of one operand
// layout (gemm_bf16.hip: LAY_NN, gemm_bf16_nt.hip, gemm_bf16_tn.hip).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace tpk {

// Launch one product with BM x BN tiles (bm 128 implies bn 128) in layout g.layout.  An
// epilogue the layout is not built for returns hipErrorInvalidValue.
hipError_t launch_shape_nn(int bm, int bn, const GemmDesc& g, hipStream_t stream);
hipError_t launch_shape_nt(int bm, int bn, const GemmDesc& g, hipStream_t stream);
hipError_t launch_shape_tn(int bm, int bn, const GemmDesc& g, hipStream_t stream);

namespace {

constexpr int BK = 32;
constexpr int NTHREADS = 256;
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
// the load) is set here and used by nothing else in the kernel.  The s_add_u32 also writes
// SCC, so SCC is declared clobbered: without it the compiler may keep a comparison result
// in SCC across this statement (seen on a K-tail bound test, which then read the carry of
// the add and loaded past K).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <uint32_t IMM>
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, i32x4_t rsrc, uint32_t soff) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
               :: "s"(lds_base), "i"(IMM), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const char* p, int second_offset) {
  const lds_char_t* lp = (const lds_char_t*)p;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lp);
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lp + second_offset));
  i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// The value unchanged, but opaque to the optimiser: a K-contiguous operand's per-lane offsets
// are the same for every tile, and without this the k-bound selections of the last K steps
// are hoisted out of the tile loop, spilled, and reloaded with a wait that also drains the
// stage loads in flight.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// GeLU, tanh form, as x / (1 + exp(-2u)) with the hardware exp2 and reciprocal (the result
// is rounded to bf16, far coarser than either approximation).
__device__ __forceinline__ float gelu_tanh_fast(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float m2log2e = -2.0f * 1.4426950408889634f;
  const float u = k0 * (x + k1 * x * x * x);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
}

// Derivative of the tanh-form GeLU.  With u = k0 (x + k1 x^3) and s = 0.5 (1 + tanh u) =
// 1 / (1 + exp(-2u)), 1 - tanh^2 u = 4 s (1 - s), so
//   gelu'(x) = s + 0.5 x (1 - tanh^2 u) u' = s (1 + 2 x (1 - s) k0 (1 + 3 k1 x^2)).
// s saturates to 0 or 1 for large |x| and the product stays finite.
__device__ __forceinline__ float gelu_tanh_grad_fast(float x) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  const float m2log2e = -2.0f * 1.4426950408889634f;
  const float x2 = x * x;
  const float u = k0 * x * (1.0f + k1 * x2);
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
  return s * (1.0f + 2.0f * k0 * x * (1.0f - s) * (1.0f + 3.0f * k1 * x2));
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

// K-contiguous operands are staged a pair of K steps at a time (see the kernel); false stages
// them one K step per ring slot like the other operands.
constexpr bool KC_PAIRS = true;

// Row permutation of the 16-byte chunks of a 128-byte LDS row of a paired operand: the 16
// lanes of a read group address 16 consecutive rows, two per 256 bytes, and (r >> 1) & 7
// sends them to 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_p(int row) { return (row >> 1) & 7; }

// Stage geometry of one operand with R rows (K-contiguous, KC) or R columns (M- or
// N-contiguous) per tile.
template <int R, bool KC>
struct OperandStage {
  static constexpr int PITCH = KC ? 64 : (R == 128 ? 256 : 512);  // bytes per LDS row
  static constexpr int BYTES = KC ? R * 64 : BK * PITCH;
  static constexpr int LD = BYTES / 4096;  // 1 KB load instructions per wave per stage
  static constexpr int CPR = PITCH / 16;   // 16-byte chunks per LDS row
  static constexpr int RPI = 1024 / PITCH; // LDS rows per load instruction
  static_assert(BYTES % 4096 == 0, "stage share must split into whole 1 KB loads per wave");
};

template <int BM, int BN, int NST, int EPI, int LAY>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmDesc g) {
  constexpr bool A_KC = (LAY & LAY_TN) == 0;  // A stored [M, K]
  constexpr bool B_KC = (LAY & LAY_NT) != 0;  // B stored as B^T [N, K]
  // A K-contiguous A operand is staged a pair of K steps at a time: pair p (steps 2p, 2p+1)
  // fills that operand's share of ring slots 2p and 2p+1 (mod NST), the first half of its
  // rows in slot 2p and the second half in slot 2p+1, each row as 128 contiguous bytes
  // (64 k).  A load then fetches whole 128-byte lines, where one K step of a row is half a
  // line: on MI355X that halves the operand's L1-to-L2 requests, and the address path had
  // stalled on them (a product whose operands are both K-contiguous ran 17 % slower than
  // the same product with neither).  Each wave's MFMA rows are one half, so a wave reads
  // one slot of the pair.
  // A pair lands about 1.5 K steps after it is issued, a single-step stage about 3 (the
  // ring holds 4 stages, so 2 pairs), so B (W^T in the input-gradient products) is staged
  // one step at a time: MI355X, same call, dY 0.971 vs 1.010 ms and dX 0.949 vs 0.975 ms
  // with both operands paired (1.03 and 1.06 ms with neither).
  constexpr bool A_PAIR = A_KC && KC_PAIRS;
  constexpr bool B_PAIR = B_KC && KC_PAIRS && LAY != LAY_NT;
  static_assert(!(A_PAIR || B_PAIR) || NST == 4, "paired staging is scheduled for a 4-slot ring");
  using SA = OperandStage<BM, A_KC>;
  using SB = OperandStage<BN, B_KC>;
  constexpr int WM = BM / 2;                      // rows per wave
  constexpr int MI = WM / 32;                     // 32-high MFMA blocks per wave
  constexpr int WN = BN / 2;                      // columns per wave
  constexpr int NJ = WN / 32;                     // 32-wide MFMA blocks per wave
  constexpr int A_BYTES = SA::BYTES;              // A's share of a stage, first
  constexpr int STAGE = A_BYTES + SB::BYTES;
  constexpr int A_LD = SA::LD;                    // load instructions per wave per stage
  constexpr int B_LD = SB::LD;                    // (paired: per half pair, the same count)
  // Per wave: LM loads per stage of the operands staged one step at a time (LMH of them go
  // out with the stage's first half), LK loads per half pair of the paired operands.  Load
  // items are numbered A first: single-step items [0, LA_M) are A's, pair items [0, LA_K).
  constexpr int LA_M = A_PAIR ? 0 : A_LD;
  constexpr int LM = LA_M + (B_PAIR ? 0 : B_LD);
  constexpr int LMH = LM / 2;
  constexpr int LA_K = A_PAIR ? A_LD : 0;
  constexpr int LK = LA_K + (B_PAIR ? B_LD : 0);
  static_assert(BN == 256 || BN == 192 || BN == 128, "tile width");
  static_assert(BM == 256 || BM == 128, "tile height");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
  // bf16 outputs leave through LDS (see the epilogue): each wave owns a 32 x WN block of
  // its own, beside the stage ring (whose slots hold the next tile's stages by then).  Not
  // with EPI_GELU_BWD: its pre-activation batch already fills the registers, and staging
  // made the compiler spill.
  constexpr bool STAGED = (EPI == EPI_STORE || EPI == EPI_GELU_TANH || EPI == EPI_GELU_SAVE) &&
                          (WN == 128 || WN == 64);
  constexpr int EPITCH = WN * 2;  // bytes per staged row
  constexpr int ECH = WN / 8;     // 16-byte chunks per staged row
  __shared__ __attribute__((aligned(16))) char epi_smem[STAGED ? 4 * 32 * EPITCH : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;

  const int64_t M = g.M, N = g.N, K = g.K;
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  // Work items: split s of output tile i is item s * ntile + i (ksplit is 1 unless the
  // launcher splits the contraction); an item contracts Kc consecutive k from s * Kc.
  const int ntile = tm * tn;
  const int nt = ntile * g.ksplit;
  const int64_t Kc = K / g.ksplit;
  const int nk = (int)((Kc + BK - 1) / BK);
  const int ng = (nk + NST - 1) / NST;  // groups of NST K steps per tile (last one padded)

  const bf16_t* __restrict__ A = (const bf16_t*)g.A;
  const bf16_t* __restrict__ B = (const bf16_t*)g.B;
  const int64_t lda = g.lda, ldb = g.ldb;

  // ---- per-lane source offsets of one tile's direct-to-LDS loads.  A K-contiguous operand's
  // instruction i of wave wv fills rows 16 (LD wv + i) .. +15 of its share, 4 lanes a row
  // (paired: rows 8 (LD wv + i) .. +7 of a half, 8 lanes a row), from a resource spanning
  // the tile's rows (k past K is sent out of range per load).  A contiguous-along-M/N
  // operand's instruction i fills k-rows RPI (LD wv + i) ..; its resource is re-based at
  // every stage (see dma_item) and columns past the end get an out-of-range offset.  A tile
  // index past the end loads zeros throughout.
  struct TileLoads {
    i32x4_t rsrc_a, rsrc_b;
    uint32_t a_off[A_LD];
    uint32_t b_off[B_LD];
    int kb;  // first k of the item's contraction range
  };
  // Row and first k (relative to the stage or pair) of lane `lane`'s 16 bytes in load
  // instruction i of a K-contiguous operand (PR: paired).
  auto kc_row = [&](auto SC, auto PC, int i) {
    using S = decltype(SC);
    return decltype(PC)::value ? 8 * (S::LD * wv + i) + (lane >> 3) : 16 * (S::LD * wv + i) + (lane >> 2);
  };
  auto kc_k = [&](auto SC, auto PC, int i) {
    const int row = kc_row(SC, PC, i);
    return 8 * (decltype(PC)::value ? (lane & 7) ^ swz_p(row) : (lane & 3) ^ swz_a(row));
  };
  // Byte offsets are formed in 32 bits: a row index below 256 times a leading dimension of
  // at most 2^21 elements (K-contiguous), or a k-row below 32 times at most 2^23, plus a
  // column below the leading dimension, stays under 2^30 bytes.
  auto kc_loads = [&](auto SC, auto PC, const bf16_t* base, int64_t rows, int64_t ld,
                      i32x4_t& rsrc, uint32_t* off) {
    using S = decltype(SC);
    rsrc = buffer_rsrc(base, rows * ld * 2);
    const uint32_t ld32 = (uint32_t)ld;
#pragma unroll
    for (int i = 0; i < S::LD; ++i)
      off[i] = ((uint32_t)kc_row(SC, PC, i) * ld32 + (uint32_t)kc_k(SC, PC, i)) * 2u;
  };
  auto tile_loads = [&](int t, TileLoads& d) {
    int tile_m = 0, tile_n = 0, ks = 0;
    const bool live = t < nt;
    if (live) {
      ks = t / ntile;
      tile_coords(t - ks * ntile, tm, tn, tile_m, tile_n);
    }
    d.kb = (int)(ks * Kc);
    const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
    if constexpr (A_KC) {
      kc_loads(SA{}, std::integral_constant<bool, A_PAIR>{}, A + m0 * lda + d.kb,
               live ? min((int64_t)BM, M - m0) : 0, lda, d.rsrc_a, d.a_off);
    } else {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int krow = SA::RPI * (A_LD * wv + i) + lane / SA::CPR;
        const int j = (lane % SA::CPR) ^ swz_b(krow);
        const int64_t m = m0 + 8 * j;
        const bool ok = live && 8 * j < BM && m < M;
        d.a_off[i] = ok ? ((uint32_t)krow * (uint32_t)lda + (uint32_t)m) * 2u : OOB;
      }
    }
    if constexpr (B_KC) {
      kc_loads(SB{}, std::integral_constant<bool, B_PAIR>{}, B + (g.n_off + n0) * ldb + d.kb,
               live ? min((int64_t)BN, N - n0) : 0, ldb, d.rsrc_b, d.b_off);
    } else {
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int krow = SB::RPI * (B_LD * wv + i) + lane / SB::CPR;
        const int j = (lane % SB::CPR) ^ swz_b(krow);
        const int64_t nlog = n0 + 8 * j;
        const bool ok = live && 8 * j < BN && nlog < N;
        // logical column of the whole B operand (below 2^23), then its physical column
        const uint32_t nb = (uint32_t)(g.n_off + nlog), blk = (uint32_t)g.b_blk;
        const uint32_t col = (nb / blk) * (uint32_t)g.b_blk_stride + nb % blk;
        d.b_off[i] = ok ? ((uint32_t)krow * (uint32_t)ldb + col) * 2u : OOB;
      }
    }
  };

  // ---- per-lane LDS fragment offsets (bytes within a stage)
  const int r32 = lane & 31, kh = lane >> 5;
  const int grp = lane >> 4, li = lane & 15, q = li & 3, s = li >> 2;
  // K-contiguous share: sub-step ks of this wave's rows w0 + 0..31 (block i adds i * 2048).
  auto kc_rd = [&](int w0, int ks) { return (w0 + r32) * 64 + (((2 * ks + kh) ^ swz_a(r32)) * 16); };
  // Paired K-contiguous share: this wave's half w of the rows (slot w of the pair), K step
  // parity par, sub-step ks (block i adds i * 4096; the pair's first slot is added at the
  // read).
  auto kp_rd = [&](int w, int par, int ks) {
    return w * STAGE + r32 * 128 + (((4 * par + 2 * ks + kh) ^ swz_p(r32)) * 16);
  };
  // Contiguous-along-M/N share: block j of this wave's columns w0.. (sub-step ks adds
  // 16 k-rows).
  auto mn_rd = [&](int w0, int j, int pitch) {
    const int chunk = w0 / 8 + 4 * j + 2 * (grp & 1) + (q >> 1);
    return (8 * (grp >> 1) + s) * pitch + ((chunk ^ swz_b(s)) * 16) + (q & 1) * 8;
  };
  int a_rd[A_PAIR ? 4 : A_KC ? 2 : MI], b_rd[B_PAIR ? 4 : B_KC ? 2 : NJ];
  if constexpr (A_PAIR) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a_rd[q] = kp_rd(wm, q >> 1, q & 1);
  } else if constexpr (A_KC) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_rd[ks] = kc_rd(wm * WM, ks);
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i) a_rd[i] = mn_rd(wm * WM, i, SA::PITCH);
  }
  if constexpr (B_PAIR) {
#pragma unroll
    for (int q = 0; q < 4; ++q) b_rd[q] = A_BYTES + kp_rd(wn, q >> 1, q & 1);
  } else if constexpr (B_KC) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) b_rd[ks] = A_BYTES + kc_rd(wn * WN, ks);
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) b_rd[j] = A_BYTES + mn_rd(wn * WN, j, SB::PITCH);
  }

  // Accumulators of the wave's WM x WN sub-tile, as MI x NJ blocks of 32 x 32.
  //   bf16 outputs (TRANS): each MFMA takes the B fragment as its first operand and the A
  //     fragment as its second, so the block it accumulates is the transpose of the output
  //     block: lane l's 16 values of block (i, j) are output row 32 i + l % 32, columns
  //     32 j + 8 q + 4 (l / 32) + 0..3 for q = 0..3, stored 8 bytes (4 bf16) at a time.
  //   fp32 outputs: A first, B second; lane l's value r of block (i, j) is output row
  //     32 i + 8 (r / 4) + 4 (l / 32) + r % 4, column 32 j + l % 32, so one 4-byte store per
  //     value writes two whole 128-byte rows per instruction.
  constexpr bool TRANS = EPI != EPI_PARTIAL_F32 && EPI != EPI_ACC_F32;
  f32x16_t acc[MI][NJ];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  };
  zero_acc();
  bf16x8_t fa[2][MI], fb[2][NJ];

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t*)smem;
  const uint32_t lds_a = lds0 + (uint32_t)(wv * A_LD * 1024);            // this wave's A loads
  const uint32_t lds_b = lds0 + (uint32_t)(A_BYTES + wv * B_LD * 1024);  // this wave's B loads

  // ---- the work items a K step is made of
  constexpr int NM = MI * NJ;  // MFMAs per half-step
  constexpr int NR = MI + NJ;  // fragment-read items per half-step
  // MFMA m of a half-step: row block m / NJ, column block m % NJ.
  auto mfma = [&](int slot, int m) {
    const int i = m / NJ, j = m % NJ;
    if constexpr (TRANS)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };
  // Read item t of sub-step ks of the stage held in buffer `buf` into fragment slot `slot`
  // (t < MI: A block t, else B block t - MI).
  auto read_item = [&](int buf, int ks, int slot, int t) {
    const char* sb = smem + buf * STAGE;
    const char* sp = smem + (buf & ~1) * STAGE;  // first slot of the pair holding stage buf
    if (t < MI) {
      if constexpr (A_PAIR) fa[slot][t] = *(const bf16x8_t*)(sp + a_rd[2 * (buf & 1) + ks] + t * 32 * 128);
      else if constexpr (A_KC) fa[slot][t] = *(const bf16x8_t*)(sb + a_rd[ks] + t * 32 * 64);
      else fa[slot][t] = ds_read_tr_pair(sb + a_rd[t] + ks * 16 * SA::PITCH, 4 * SA::PITCH);
    } else {
      const int j = t - MI;
      if constexpr (B_PAIR) fb[slot][j] = *(const bf16x8_t*)(sp + b_rd[2 * (buf & 1) + ks] + j * 32 * 128);
      else if constexpr (B_KC) fb[slot][j] = *(const bf16x8_t*)(sb + b_rd[ks] + j * 32 * 64);
      else fb[slot][j] = ds_read_tr_pair(sb + b_rd[j] + ks * 16 * SB::PITCH, 4 * SB::PITCH);
    }
  };
  // Single-step load item U of stage kd (counted within the tile whose loads `d` describes)
  // into buffer BUF (U < LA_M: an A load, else a B load).  Parts of a stage past K, and
  // whole stages past K, come back as zeros (out-of-range offsets or an empty range), so the
  // K loop can run whole groups of NST steps.  A contiguous-along-M/N operand's resource is
  // re-based at every stage so that its range check alone bounds the k-rows read; a
  // K-contiguous operand's k bound is tested per lane, in a step (or pair) that reaches past K
  // (the test is wave-uniform otherwise), and only in loads issued in the last two groups of
  // K steps of a tile (CHK): an earlier load's stage ends at or before K.
  const int Ki = (int)Kc;                      // K < 2^31 (bounded by the leading dimensions)
  const int lda2 = (int)(lda * 2), ldb2 = (int)(ldb * 2);  // bytes per stored row
  const char* const Abytes = (const char*)A;
  const char* const Bbytes = (const char*)B;
  auto dma_item = [&](auto CHKC, auto BUFC, auto UC, const TileLoads& d, int kd) {
    constexpr bool CHK = decltype(CHKC)::value;
    constexpr int BUF = decltype(BUFC)::value, U = decltype(UC)::value;
    const int k0 = kd * BK;
    if constexpr (U < LA_M) {
      if constexpr (A_KC) {
        uint32_t off = d.a_off[U];
        if constexpr (CHK) {
          off = opaque(off);
          if (k0 + BK > Ki && kc_k(SA{}, std::false_type{}, U) >= Ki - k0) off = OOB;
        }
        dma16<BUF * STAGE + U * 1024>(lds_a, off, d.rsrc_a, (uint32_t)k0 * 2u);
      } else {
        const int k_rows = max(0, min(BK, Ki - k0));
        const i32x4_t rsrc = buffer_rsrc(Abytes + (int64_t)(d.kb + k0) * lda2, (int64_t)(k_rows * lda2));
        dma16<BUF * STAGE + U * 1024>(lds_a, d.a_off[U], rsrc, 0u);
      }
    } else {
      constexpr int I = U - LA_M;
      if constexpr (B_KC) {
        uint32_t off = d.b_off[I];
        if constexpr (CHK) {
          off = opaque(off);
          if (k0 + BK > Ki && kc_k(SB{}, std::false_type{}, I) >= Ki - k0) off = OOB;
        }
        dma16<BUF * STAGE + I * 1024>(lds_b, off, d.rsrc_b, (uint32_t)k0 * 2u);
      } else {
        const int k_rows = max(0, min(BK, Ki - k0));
        const i32x4_t rsrc = buffer_rsrc(Bbytes + (int64_t)(d.kb + k0) * ldb2, (int64_t)(k_rows * ldb2));
        dma16<BUF * STAGE + I * 1024>(lds_b, d.b_off[I], rsrc, 0u);
      }
    }
  };
  // Pair load item U (U < LA_K: A, else B) of half H of pair kp into slot BUF (the pair's
  // first slot + H); k past K comes back as zeros.  The second half's rows are reached by
  // moving the resource's base by half a tile of rows (and shrinking its range to match),
  // so both halves share the per-lane offsets.
  const uint32_t a_half = (uint32_t)((BM / 2) * lda * 2), b_half = (uint32_t)((BN / 2) * ldb * 2);
  auto second_half = [](i32x4_t r, uint32_t bytes) {
    const uint64_t base = ((uint64_t)(uint32_t)r.y << 32 | (uint32_t)r.x) + bytes;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)((uint32_t)r.z > bytes ? (uint32_t)r.z - bytes : 0u));
    return r;
  };
  auto dma_pair = [&](auto CHKC, auto BUFC, auto HC, auto UC, const TileLoads& d, int kp) {
    constexpr bool CHK = decltype(CHKC)::value;
    constexpr int BUF = decltype(BUFC)::value, H = decltype(HC)::value, U = decltype(UC)::value;
    const int k0 = kp * 2 * BK;
    if constexpr (U < LA_K) {
      uint32_t off = d.a_off[U];
      if constexpr (CHK) {
        off = opaque(off);
        if (k0 + 2 * BK > Ki && kc_k(SA{}, std::true_type{}, U) >= Ki - k0) off = OOB;
      }
      dma16<BUF * STAGE + U * 1024>(lds_a, off, H ? second_half(d.rsrc_a, a_half) : d.rsrc_a,
                                    (uint32_t)k0 * 2u);
    } else {
      constexpr int I = U - LA_K;
      uint32_t off = d.b_off[I];
      if constexpr (CHK) {
        off = opaque(off);
        if (k0 + 2 * BK > Ki && kc_k(SB{}, std::true_type{}, I) >= Ki - k0) off = OOB;
      }
      dma16<BUF * STAGE + I * 1024>(lds_b, off, H ? second_half(d.rsrc_b, b_half) : d.rsrc_b,
                                    (uint32_t)k0 * 2u);
    }
  };

  // One half-step: the NM MFMAs on fragment slot SLOT, with, spread between them and each
  // fenced in place, NR fragment reads (sub-step ks_read of buffer RBUF into slot
  // read_slot), then NK pair loads (half PH of pair kd / 2, into slot PBUF), then the
  // single-step load items [LO, HI) of stage kd (into buffer DBUF).
  auto half_step = [&](auto CHKC, auto SLOTC, auto LOC, auto HIC, auto NKC, auto PHC, auto PBUFC,
                       auto RBUFC, int ks_read, int read_slot, auto DBUFC, const TileLoads& d,
                       int kd) {
    constexpr int SLOT = decltype(SLOTC)::value;
    constexpr int LO = decltype(LOC)::value, HI = decltype(HIC)::value;
    constexpr int NK = decltype(NKC)::value;
    constexpr int RBUF = decltype(RBUFC)::value;
    constexpr int NITEM = NR + NK + (HI - LO);
    static_for<NM>([&](auto MC) {
      constexpr int m = decltype(MC)::value;
      mfma(SLOT, m);
      __builtin_amdgcn_sched_barrier(0);
      static_for<NITEM>([&](auto TC) {
        constexpr int t = decltype(TC)::value;
        if constexpr (t * NM / NITEM == m) {
          if constexpr (t < NR) read_item(RBUF, ks_read, read_slot, t);
          else if constexpr (t < NR + NK)
            dma_pair(CHKC, PBUFC, PHC, std::integral_constant<int, t - NR>{}, d, kd >> 1);
          else dma_item(CHKC, DBUFC, std::integral_constant<int, LO + t - NR - NK>{}, d, kd);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // One K step on the stage in buffer S.  First half: the MFMAs of sub-step 0, with the
  // reads of sub-step 1 and the second half of the loads of the stage NST-1 ahead (into
  // buffer S-1, free since the previous step's barrier) between them.  Then the wait for
  // this wave's loads of the next stage (the NST-2 stages after it may still be in flight)
  // and the barrier, after which every wave's share of the next stage has landed and buffer
  // S is no longer read.  Second half: the MFMAs of sub-step 1, with the reads of the next
  // stage's sub-step 0 and the first half of the loads of the stage NST ahead (into buffer
  // S) between them.  Splitting each stage's loads over two half-steps keeps the four waves'
  // 1 KB loads from reaching the address unit in one burst.
  // Paired operands: pair p's slots are free after the barrier of step 2p - 3 and must hold
  // it by the barrier of step 2p - 1, so its first half goes out in the second half of step
  // 2p - 3 (beside the first half of stage 2p + 1) and its second half in the first half of
  // step 2p - 2 (beside the second half of stage 2p + 1): a half-step that loads an odd
  // stage kd also loads a half of pair kd / 2.  The waits count this wave's loads issued
  // after the last one the next step reads (pair loads go out before the single-step ones
  // of the same half-step): at an even step that is the second half of stage S + 1, with
  // 2 LM + 2 LK loads after it; at an odd step the second half of the pair holding S + 1,
  // issued one step earlier, with 2 LM - LMH after it.
  using std::integral_constant;
  auto step = [&](auto SC, auto CHKC, const TileLoads& d1, int kd1, const TileLoads& d2, int kd2) {
    constexpr int S = decltype(SC)::value;
    constexpr int SL1 = (S + NST - 1) % NST;                   // slot of stage kd1
    constexpr bool P1 = LK > 0 && (S + NST - 1) % 2 == 1;     // kd1 odd
    constexpr bool P2 = LK > 0 && S % 2 == 1;                 // kd2 = kd1 + 1 odd
    constexpr int WAIT = LK == 0 ? (NST - 2) * LM : S % 2 == 0 ? 2 * LM + 2 * LK : 2 * LM - LMH;
    half_step(CHKC, integral_constant<int, 0>{}, integral_constant<int, LMH>{}, integral_constant<int, LM>{},
              integral_constant<int, P1 ? LK : 0>{}, integral_constant<int, 1>{},
              integral_constant<int, (SL1 & ~1) + 1>{}, SC, 1, 1, integral_constant<int, SL1>{}, d1, kd1);
    wait_vmcnt_lgkm0<WAIT>();
    lds_barrier();
    half_step(CHKC, integral_constant<int, 1>{}, integral_constant<int, 0>{}, integral_constant<int, LMH>{},
              integral_constant<int, P2 ? LK : 0>{}, integral_constant<int, 0>{},
              integral_constant<int, S & ~1>{}, integral_constant<int, (S + 1) % NST>{}, 0, 0, SC,
              d2, kd2);
  };

  // ---- persistent loop over this workgroup's tiles t = blockIdx.x + i * gridDim.x.  The
  // stage stream runs on across tiles: the last group of K steps of a tile loads the first
  // stages of the next one, so the loads are in flight during the epilogue.
  TileLoads cur, nxt;
  int t = blockIdx.x;
  tile_loads(t, cur);
  // prologue: stages 0 .. NST-2 and the first half of stage NST-1 in flight (its second
  // half goes out in the first step), pair 0 and the first half of pair 1 likewise, in the
  // order pair 0, stage 0, stage 1, half of pair 1, stage 2, half of stage 3; stage 0 and
  // pair 0 landed, their first fragments read
  const std::true_type chk;
  if constexpr (LK > 0) {
    static_for<LK>([&](auto UC) { dma_pair(chk, integral_constant<int, 0>{}, integral_constant<int, 0>{}, UC, cur, 0); });
    static_for<LK>([&](auto UC) { dma_pair(chk, integral_constant<int, 1>{}, integral_constant<int, 1>{}, UC, cur, 0); });
  }
  static_for<NST - 1>([&](auto SC) {
    static_for<LM>([&](auto UC) { dma_item(chk, SC, UC, cur, decltype(SC)::value); });
    if constexpr (LK > 0 && decltype(SC)::value == 1)
      static_for<LK>([&](auto UC) { dma_pair(chk, integral_constant<int, 2>{}, integral_constant<int, 0>{}, UC, cur, 1); });
  });
  static_for<LMH>([&](auto UC) { dma_item(chk, integral_constant<int, NST - 1>{}, UC, cur, NST - 1); });
  wait_vmcnt<LK == 0 ? (NST - 2) * LM + LMH : 2 * LM + LK + LMH>();
  lds_barrier();
#pragma unroll
  for (int r = 0; r < NR; ++r) read_item(0, 0, 0, r);

  const int64_t ldc = g.ldc;
  for (; t < nt; t += gridDim.x) {
    tile_loads(t + gridDim.x, nxt);
    // Groups 0 .. ng-3 load stages that end at or before K (unchecked); group ng-2 loads the
    // last group's stages and the last group the next tile's first ones (checked).
    auto group = [&](auto CHKC, int gi) {
      const int kt = gi * NST;
      static_for<NST>([&](auto SC) {
        constexpr int S = decltype(SC)::value;
        step(SC, CHKC, cur, kt + S + NST - 1, cur, kt + S + NST);
      });
    };
    for (int gi = 0; gi < ng - 2; ++gi) group(std::false_type{}, gi);
    if (ng >= 2) group(chk, ng - 2);
    {  // last group: from its first second half on, the loads are the next tile's
      const int kt = (ng - 1) * NST;
      step(std::integral_constant<int, 0>{}, chk, cur, kt + NST - 1, nxt, 0);
      static_for<NST - 1>([&](auto SC) {
        constexpr int S = decltype(SC)::value + 1;
        step(std::integral_constant<int, S>{}, chk, nxt, S - 1, nxt, S);
      });
    }

    // Epilogue of item t (see the accumulator layout above).
    int tile_m, tile_n;
    const int ks = t / ntile;
    tile_coords(t - ks * ntile, tm, tn, tile_m, tile_n);
    const int64_t m_w = (int64_t)tile_m * BM + wm * WM, n_w = (int64_t)tile_n * BN + wn * WN;
    if constexpr (TRANS) {
      const int64_t row0 = m_w + (lane & 31), col0 = n_w + 4 * (lane >> 5);
      // EPI_GELU_BWD: the tile's pre-activation values, all loaded before the first store.
      // Loads and stores share one completion counter and complete out of order with
      // respect to each other, so a load still pending behind a store can only be waited
      // for with the store; one batch of loads and one wait keeps the stores from
      // serialising the epilogue.
      uint2 pre[EPI == EPI_GELU_BWD ? MI : 1][EPI == EPI_GELU_BWD ? NJ : 1][4];
      if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int64_t row = row0 + 32 * i, col = col0 + 32 * j + 8 * qq;
              pre[i][j][qq] = row < M && col < N
                                  ? *(const uint2*)((const bf16_t*)g.aux + row * g.ldaux + col)
                                  : make_uint2(0u, 0u);
            }
        // One explicit wait for the whole batch: the bounds-checked stores below branch, and
        // without it the compiler waits for every earlier store before each use of a value.
        wait_vmcnt<0>();
      }
      // Item (i, j, qq) of the lane: output row 32 i + lane % 32 (of the wave's block), columns
      // 32 j + 8 qq + 4 (lane / 32) + 0..3, as 4 packed bf16; the pre-activation (raw
      // accumulator) for the saved copy of EPI_GELU_SAVE.
      auto item = [&](int i, int j, int qq, bool raw) {
        float v0 = acc[i][j][4 * qq], v1 = acc[i][j][4 * qq + 1];
        float v2 = acc[i][j][4 * qq + 2], v3 = acc[i][j][4 * qq + 3];
        if (!raw) {
          if constexpr (EPI == EPI_GELU_TANH || EPI == EPI_GELU_SAVE) {
            v0 = gelu_tanh_fast(v0); v1 = gelu_tanh_fast(v1);
            v2 = gelu_tanh_fast(v2); v3 = gelu_tanh_fast(v3);
          }
          if constexpr (EPI == EPI_GELU_BWD) {
            const uint2 p = pre[i][j][qq];
            v0 *= gelu_tanh_grad_fast(__uint_as_float(p.x << 16));
            v1 *= gelu_tanh_grad_fast(__uint_as_float(p.x & 0xFFFF0000u));
            v2 *= gelu_tanh_grad_fast(__uint_as_float(p.y << 16));
            v3 *= gelu_tanh_grad_fast(__uint_as_float(p.y & 0xFFFF0000u));
          }
        }
        uint2 u;
        u.x = pack_bf16x2(v0, v1);
        u.y = pack_bf16x2(v2, v3);
        return u;
      };
      if constexpr (STAGED) {
        // Through LDS: a lane's items cover 16 bytes of each of 32 rows, so stored directly
        // every store instruction would touch 32 rows with 16 bytes each.  Row block i of the
        // wave is written to its LDS block in that layout and read back as whole 16-byte
        // chunks, 64 / ECH rows per instruction, so each global store writes 64 / ECH rows of
        // WN * 2 contiguous bytes.  Chunk c of staged row r sits at chunk (c + r) mod ECH,
        // which spreads a write's 32 rows over the LDS banks.  The block is private to the
        // wave and its LDS accesses execute in order, so no barrier is needed.
        char* const ew = epi_smem + wv * (32 * EPITCH);
        const int er = lane & 31, eh = lane >> 5;
        constexpr int RPI_E = 64 / ECH;
        const int rr = lane / ECH, ch = lane % ECH;
        auto staged = [&](int i, bool raw, void* dst, int64_t ld) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int c = (4 * j + qq + er) & (ECH - 1);
              *(uint2*)(ew + er * EPITCH + c * 16 + eh * 8) = item(i, j, qq, raw);
            }
#pragma unroll
          for (int it = 0; it < 32 / RPI_E; ++it) {
            const int r = it * RPI_E + rr;
            const uint4 v = *(const uint4*)(ew + r * EPITCH + ((ch + r) & (ECH - 1)) * 16);
            const int64_t row = m_w + 32 * i + r, col = n_w + 8 * ch;
            if (row < M && col < N) *(uint4*)((bf16_t*)dst + row * ld + col) = v;
          }
        };
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if constexpr (EPI == EPI_GELU_SAVE) staged(i, true, g.aux, g.ldaux);
          staged(i, false, g.C, ldc);
        }
      } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int64_t row = row0 + 32 * i;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int64_t col = col0 + 32 * j + 8 * qq;
              if (row < M && col < N) {
                if constexpr (EPI == EPI_GELU_SAVE)
                  *(uint2*)((bf16_t*)g.aux + row * g.ldaux + col) = item(i, j, qq, true);
                *(uint2*)((bf16_t*)g.C + row * ldc + col) = item(i, j, qq, false);
              }
            }
          }
        }
      }
    } else {
      const int64_t row0 = m_w + 4 * (lane >> 5), col0 = n_w + (lane & 31);
      float* const Cs = (float*)g.C + (int64_t)ks * g.c_split_stride;  // this split's partial
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        // EPI_ACC_F32: row block i's previous values in one batch of loads, then the stores
        // (one wait per row block rather than per value, as for the pre-activation above).
        float old[EPI == EPI_ACC_F32 ? NJ : 1][16];
        if constexpr (EPI == EPI_ACC_F32) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t row = row0 + 32 * i + 8 * (r >> 2) + (r & 3), col = col0 + 32 * j;
              old[j][r] = row < M && col < N ? ((const float*)g.C)[row * ldc + col] : 0.0f;
            }
          wait_vmcnt<0>();
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int64_t col = col0 + 32 * j;
          if constexpr (EPI == EPI_ACC_F32) {
            // The block's previous values were read with the rest of row block i (below).
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
              if (row < M && col < N) ((float*)g.C)[row * ldc + col] = old[j][r] + acc[i][j][r];
            }
          } else {
            // Streaming stores: a partial is read once, by a later kernel, and a product's
            // partials outgrow every cache level; dirty lines left in the Infinity Cache would
            // be written back during the reduce that reads the partials (on MI355X these stores
            // take the reduce after the product from 730 to 712 us, and the product itself
            // from 913 to 907 us).
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
              if (row < M && col < N) __builtin_nontemporal_store(acc[i][j][r], Cs + row * ldc + col);
            }
          }
        }
      }
    }
    zero_acc();
    cur = nxt;
  }
  // Loads of the stages past the last tile are still in flight: let them land before the
  // workgroup's LDS is released.
  wait_vmcnt<0>();
}

// Epilogues built for each operand layout.
template <int LAY, int EPI>
constexpr bool layout_has_epilogue() {
  if (LAY == LAY_NN) return EPI == EPI_STORE || EPI == EPI_GELU_TANH || EPI == EPI_PARTIAL_F32 ||
                            EPI == EPI_GELU_SAVE || EPI == EPI_ACC_F32;
  if (LAY == LAY_NT) return EPI == EPI_STORE || EPI == EPI_GELU_BWD || EPI == EPI_PARTIAL_F32;
  if (LAY == LAY_TN) return EPI == EPI_PARTIAL_F32 || EPI == EPI_ACC_F32;
  return false;
}

template <int BM, int BN, int NST, int LAY, int EPI>
hipError_t launch_epi(dim3 grid, const GemmDesc& g, hipStream_t stream) {
  if constexpr (layout_has_epilogue<LAY, EPI>()) {
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, NST, EPI, LAY>), grid, dim3(NTHREADS), 0, stream, g);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int BM, int BN, int NST, int LAY>
hipError_t launch_tile(const GemmDesc& g, hipStream_t stream) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  const int64_t tiles = tm * tn * g.ksplit;  // work items
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  // One workgroup per compute unit (each holds 64-128 KB of LDS), looping over tiles.
  const int64_t blocks = min(tiles, (int64_t)device_cus());
  const dim3 grid((unsigned)blocks);
  switch (g.epi) {
    case EPI_STORE: return launch_epi<BM, BN, NST, LAY, EPI_STORE>(grid, g, stream);
    case EPI_GELU_TANH: return launch_epi<BM, BN, NST, LAY, EPI_GELU_TANH>(grid, g, stream);
    case EPI_PARTIAL_F32: return launch_epi<BM, BN, NST, LAY, EPI_PARTIAL_F32>(grid, g, stream);
    case EPI_GELU_SAVE: return launch_epi<BM, BN, NST, LAY, EPI_GELU_SAVE>(grid, g, stream);
    case EPI_GELU_BWD: return launch_epi<BM, BN, NST, LAY, EPI_GELU_BWD>(grid, g, stream);
    case EPI_ACC_F32: return launch_epi<BM, BN, NST, LAY, EPI_ACC_F32>(grid, g, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int LAY>
hipError_t launch_shape_t(int bm, int bn, const GemmDesc& g, hipStream_t stream) {
  if (g.layout != LAY) return hipErrorInvalidValue;
  if (bm == 128) return launch_tile<128, 128, 4, LAY>(g, stream);
  switch (bn) {
    case 192: return launch_tile<256, 192, 4, LAY>(g, stream);
    case 128: return launch_tile<256, 128, 4, LAY>(g, stream);
    default: return launch_tile<256, 256, 4, LAY>(g, stream);
  }
}

}  // namespace
}  // namespace tpk
