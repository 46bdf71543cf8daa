// Partial reduce + residual + LayerNorm, the in-HBM replacement of the tensor-parallel
// all-reduce (pwwt.cn TP walk-through section 2.3: the all-reduce sits just before the
// residual add and can be fused with it and with the next LayerNorm's statistics; section
// 6.3: residual + LayerNorm as one fused op with one fixed statistics order).
//
//   h = residual + sum_{p ascending} parts[p];  y = (h - mean) / sqrt(var + eps) * gamma + beta
//
// HBM-bound.  One workgroup per row at a time; each thread owns NCH runs of 8 elements.  In a
// full row (the runs fill it exactly) that is not summed from bf16 partials, a run is two
// halves of 4 consecutive elements 256 apart (lane l of wave w holds elements 4l.. and
// 256 + 4l.. of the wave's 512-element segment), so every load and store instruction of a
// wave covers one contiguous range: 64 x 16 bytes of an fp32 partial.  Eight consecutive elements per lane would leave each 16-byte load touching every
// other 16 bytes of a 2 KB span, and a row sum of 8 fp32 partials over that layout measured 7 to
// 10 % slower on MI355X.  Otherwise (bf16 partials, ragged rows) a run is 8 consecutive elements
// (16 bytes of a bf16 row), runs spaced THREADS apart.  The partials are read in two alternating register batches
// (partial p+1 in flight while p is added); then the residual row; then gamma and beta ahead
// of the statistics.  The partials are read once and the outputs written once, so those
// accesses are streaming (non-temporal): on MI355X that moves the fused reduce from 4.9 to
// 5.45 TB/s.  A streaming residual load measured slower and is not used, and so did every
// other cache policy of the output stores.  Writing h alone instead of h and y (0.2 GB less
// for the block's 8192 x 12288 reduce of 8 partials) takes 649 instead of 669 us on MI355X.
// The row stays in registers: the mean is a wave shuffle reduction plus one cross-wave step
// through LDS, and the variance is a second pass over the registers (no E[x^2] - mean^2).
#include <atomic>

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

struct F8 {
  float v[8];
};

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// Cache policy of a buffer load: non-temporal (streaming; the partials are read once).
constexpr int CPOL_NT = 2;

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// 8 consecutive elements of a bf16 or fp32 output row, written as streaming stores.
template <bool BF16>
__device__ __forceinline__ void store8(void* p, int64_t idx, const F8& r) {
  if (BF16) {
    const u32x4_t u = {pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3]),
                       pack_bf16x2(r.v[4], r.v[5]), pack_bf16x2(r.v[6], r.v[7])};
    __builtin_nontemporal_store(u, (u32x4_t*)((bf16_t*)p + idx));
  } else {
    __builtin_nontemporal_store(f32x4_t{r.v[0], r.v[1], r.v[2], r.v[3]}, (f32x4_t*)((float*)p + idx));
    __builtin_nontemporal_store(f32x4_t{r.v[4], r.v[5], r.v[6], r.v[7]}, (f32x4_t*)((float*)p + idx + 4));
  }
}

// Raw 16 bytes (8 bf16) or 32 bytes (8 fp32) of a row, loaded as one batch item.
template <bool BF16>
struct Raw8;
template <>
struct Raw8<true> {
  uint4 u;
};
template <>
struct Raw8<false> {
  f32x4_t a, b;
};

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void* p, int64_t idx) {
  Raw8<BF16> r;
  if constexpr (BF16) {
    r.u = *(const uint4*)((const bf16_t*)p + idx);
  } else {
    r.a = *(const f32x4_t*)((const float*)p + idx);
    r.b = *(const f32x4_t*)((const float*)p + idx + 4);
  }
  return r;
}

// A run of reduce_ln_kernel: elements idx .. idx+3 and idxb .. idxb+3 (idxb = idx + 4 unless
// SPLIT), loaded into / stored from the 8 values in that order.
template <bool BF16, bool SPLIT>
__device__ __forceinline__ Raw8<BF16> load_run(const void* p, int64_t idx, int64_t idxb) {
  if constexpr (BF16 && SPLIT) {
    Raw8<BF16> r;
    const uint2 a = *(const uint2*)((const bf16_t*)p + idx);
    const uint2 b = *(const uint2*)((const bf16_t*)p + idxb);
    r.u = make_uint4(a.x, a.y, b.x, b.y);
    return r;
  } else if constexpr (BF16) {
    return load_raw8<true>(p, idx);
  } else {
    Raw8<BF16> r;
    r.a = *(const f32x4_t*)((const float*)p + idx);
    r.b = *(const f32x4_t*)((const float*)p + idxb);
    return r;
  }
}

template <bool BF16, bool SPLIT>
__device__ __forceinline__ void store_run(void* p, int64_t idx, int64_t idxb, const F8& r) {
  if constexpr (BF16 && SPLIT) {
    __builtin_nontemporal_store(u32x2_t{pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3])},
                                (u32x2_t*)((bf16_t*)p + idx));
    __builtin_nontemporal_store(u32x2_t{pack_bf16x2(r.v[4], r.v[5]), pack_bf16x2(r.v[6], r.v[7])},
                                (u32x2_t*)((bf16_t*)p + idxb));
  } else if constexpr (BF16) {
    store8<true>(p, idx, r);
  } else {
    __builtin_nontemporal_store(f32x4_t{r.v[0], r.v[1], r.v[2], r.v[3]}, (f32x4_t*)((float*)p + idx));
    __builtin_nontemporal_store(f32x4_t{r.v[4], r.v[5], r.v[6], r.v[7]}, (f32x4_t*)((float*)p + idxb));
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float* v) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = r.a[e];
      v[4 + e] = r.b[e];
    }
  }
}

// FULL: every run of every thread lies inside the row (H == NCH * THREADS * 8), so no run
// needs a bounds test and each batch of loads is issued without branches.
// PARTS: n_parts > 0; RES: a residual is given; LN: gamma is given (the LayerNorm runs).  They
// are compile-time so that the row loop has no data-dependent branch around its loads: at
// such a join the compiler waits for every load in flight, which would include the next
// row's prefetched partial.
// PB: the partials are bf16 (16 bytes per run of 8), summed in fp32 exactly as fp32 ones.
template <int THREADS, int NCH, bool BF16, bool FULL, bool PARTS, bool RES, bool LN, bool PB = false>
__global__ __launch_bounds__(THREADS) void reduce_ln_kernel(ReduceDesc r) {
  __shared__ float red[THREADS / 64];
  const int tid = threadIdx.x;
  const int64_t H = r.H;
  // SPLIT: each run is two 4-element halves, 256 elements apart (see the top of the file); a
  // ragged row keeps 8 consecutive elements per run, so one bounds test covers the run.
  constexpr bool SPLIT = FULL && !PB;
  bool in[NCH];
  int64_t col[NCH], colb[NCH];  // first element of each half of the run
  uint32_t boff[NCH], boffb[NCH];  // their byte offsets in an fp32 row (past the row: out of range)
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if constexpr (SPLIT) {
      col[c] = ((int64_t)c * (THREADS / 64) + (tid >> 6)) * 512 + 4 * (tid & 63);
      colb[c] = col[c] + 256;
    } else {
      col[c] = ((int64_t)c * THREADS + tid) * 8;
      colb[c] = col[c] + 4;
    }
    in[c] = FULL || col[c] < H;
    boff[c] = (uint32_t)col[c] * 4u;
    boffb[c] = (uint32_t)colb[c] * 4u;
  }
  const int np = r.n_parts;
  // Partial p of row `row` into batch q: buffer loads from a resource spanning that row of the
  // partial (wave-uniform, in scalar registers), at per-lane byte offsets shared by all
  // partials; a row past the last has an empty range and reads as zeros.
  // (bf16 partials: the 16 bytes of a run in q[c][0], as raw bits)
  constexpr int PES = PB ? 2 : 4;  // bytes per element of a partial
  auto load_part = [&](int64_t row, int p, f32x4_t (&q)[NCH][2]) __attribute__((always_inline)) {
    const bool ok = row < r.rows;
    const char* part = (const char*)r.parts + (ok ? ((int64_t)p * r.part_stride + row * H) * PES : 0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)part, (short)0, ok ? (int)(H * PES) : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (PB) {
        q[c][0] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[c] / 2, 0, CPOL_NT));
      } else {
        q[c][0] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[c], 0, CPOL_NT));
        q[c][1] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, boffb[c], 0, CPOL_NT));
      }
    }
  };
  // gamma and beta: for bf16 rows of up to 2048 runs they are loaded once per workgroup into
  // LDS, where each thread reads back only the runs it wrote (per-thread storage: no barrier,
  // 16 consecutive bytes per lane, no bank conflict); that keeps them out of the registers
  // that hold the next row's prefetched partial.  Otherwise they are loaded per row.
  constexpr bool GB_LDS = LN && BF16 && NCH * THREADS <= 2048;
  __shared__ Raw8<BF16> gb_lds[GB_LDS ? 2 : 1][GB_LDS ? NCH * THREADS : 1];
  if constexpr (GB_LDS) {
    const void* beta = r.beta ? r.beta : r.gamma;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      Raw8<BF16> g{}, b{};
      if (in[c]) {
        g = load_run<BF16, SPLIT>(r.gamma, col[c], colb[c]);
        b = load_run<BF16, SPLIT>(beta, col[c], colb[c]);
      }
      gb_lds[0][c * THREADS + tid] = g;
      gb_lds[1][c * THREADS + tid] = b;
    }
  }
  // Partial 0 of the workgroup's next row is loaded before the current row's residual,
  // statistics and stores, so the row's tail never leaves the workgroup with no read in
  // flight (the first row's comes before the loop).
  f32x4_t qa[NCH][2], qb[NCH][2];
  if constexpr (PARTS) load_part(blockIdx.x, 0, qa);
  for (int64_t row = blockIdx.x; row < r.rows; row += gridDim.x) {
    const int64_t roff = row * H;                              // inputs: dense rows
    const int64_t ooff = row * (r.ld_out > 0 ? r.ld_out : H);  // outputs: rows of pitch ld_out

    // h = sum of the partials in ascending order, then + residual.  Two register batches
    // alternate: the loads of partial p+1 go out before partial p is added, so one batch is
    // always in flight while the other is summed.  The loop body has no branch: a conditional
    // use of a batch lets the compiler sink its loads behind the next batch's and wait for
    // both; the last one or two partials are summed after it.
    float v[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
    auto add_part = [&](const f32x4_t (&q)[NCH][2]) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if constexpr (PB) {
          Raw8<true> raw;
          raw.u = __builtin_bit_cast(uint4, q[c][0]);
          float x[8];
          unpack8<true>(raw, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += x[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[c][e] += q[c][0][e];
            v[c][4 + e] += q[c][1][e];
          }
        }
      }
    };
    if constexpr (PARTS) {
      // The scheduling barriers keep each batch's loads ahead of the previous batch's adds
      // (the scheduler would otherwise move the adds up and wait with nothing in flight).
      int p = 0;
      for (; p + 2 < np; p += 2) {
        load_part(row, p + 1, qb);
        __builtin_amdgcn_sched_barrier(0);
        add_part(qa);
        __builtin_amdgcn_sched_barrier(0);
        load_part(row, p + 2, qa);
        __builtin_amdgcn_sched_barrier(0);
        add_part(qb);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (p + 1 < np) {
        load_part(row, p + 1, qb);
        __builtin_amdgcn_sched_barrier(0);
        add_part(qa);
        __builtin_amdgcn_sched_barrier(0);
        add_part(qb);
      } else {
        add_part(qa);
      }
    }
    // The row's other loads (residual, gamma, beta) go out before the next row's first partial:
    // the vector-memory counter completes in order, so waiting for a load issued after the
    // prefetch would also wait for the prefetch.  beta NULL reads gamma's values and uses 0.
    Raw8<BF16> res[NCH];
    if constexpr (RES) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (in[c]) res[c] = load_run<BF16, SPLIT>(r.residual, roff + col[c], roff + colb[c]);
    }
    Raw8<BF16> gm[NCH], bt[NCH];
    if constexpr (LN && !GB_LDS) {
      const void* beta = r.beta ? r.beta : r.gamma;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (in[c]) {
          gm[c] = load_run<BF16, SPLIT>(r.gamma, col[c], colb[c]);
          bt[c] = load_run<BF16, SPLIT>(beta, col[c], colb[c]);
        }
      }
    }
    if constexpr (PARTS) {
      __builtin_amdgcn_sched_barrier(0);
      load_part(row + gridDim.x, 0, qa);
      __builtin_amdgcn_sched_barrier(0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (in[c]) {
        if constexpr (RES) {
          float x[8];
          unpack8<BF16>(res[c], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += x[e];
        }
        if (r.h_out) {
          F8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o.v[e] = v[c][e];
          store_run<BF16, SPLIT>(r.h_out, ooff + col[c], ooff + colb[c], o);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) sum += v[c][e] + v[c][e + 1];
    }
    if constexpr (!LN) continue;
    const float inv_h = 1.0f / (float)H;
    const float mean = block_sum<THREADS>(sum, red) * inv_h;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (in[c]) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float a0 = v[c][e] - mean, a1 = v[c][e + 1] - mean;
          sq += a0 * a0 + a1 * a1;
        }
      }
    }
    const float var = block_sum<THREADS>(sq, red) * inv_h;
    const float rstd = 1.0f / sqrtf(var + r.eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (in[c]) {
        float gv[8], bv[8];
        if constexpr (GB_LDS) {
          unpack8<BF16>(gb_lds[0][c * THREADS + tid], gv);
          unpack8<BF16>(gb_lds[1][c * THREADS + tid], bv);
        } else {
          unpack8<BF16>(gm[c], gv);
          unpack8<BF16>(bt[c], bv);
        }
        if (!r.beta)
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
        F8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y.v[e] = (v[c][e] - mean) * rstd * gv[e] + bv[e];
        store_run<BF16, SPLIT>(r.y_out, ooff + col[c], ooff + colb[c], y);
      }
    }
  }  // row loop
}

// The same operation with no partials to sum (h = residual; the pre-attention LayerNorm of
// the block).  A workgroup loops over rows blockIdx.x, + gridDim.x, ... and issues the loads of
// its next row before it starts on the current one, so every workgroup keeps one row's reads in
// flight through its reductions and stores.  Three raw row buffers rotate (the loop is
// unrolled three times), so no register copy waits on a load in flight; the row is unpacked again
// for each of its three passes (sum, squares, output) instead of being held as fp32, and gamma
// and beta are loaded once per workgroup into LDS.  That keeps the registers per workgroup low
// and the rows in flight per compute unit high.  Every load of a row is issued before the previous
// row's wait (the vector-memory counter completes in order, so a later load that the current
// row waited on would also wait for the prefetch).  The row loads are buffer loads from a
// resource spanning that row (none past the last row: such a resource has no bytes in range
// and its loads return zeros), so the prefetch needs no branch.  The statistics are taken in
// the order of reduce_ln_kernel.
template <int THREADS, int NCH, bool BF16, bool FULL>
__global__ __launch_bounds__(THREADS) void ln_rows_kernel(ReduceDesc r) {
  __shared__ float red[THREADS / 64];
  const int tid = threadIdx.x;
  const int64_t H = r.H;
  constexpr int ES = BF16 ? 2 : 4;
  uint32_t boff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) boff[c] = (uint32_t)((c * THREADS + tid) * 8 * ES);
  auto in = [&](int c) { return FULL || (int64_t)(c * THREADS + tid) * 8 < H; };
  const bool ln = r.gamma != nullptr, has_beta = r.beta != nullptr, has_h = r.h_out != nullptr;
  // gamma and beta, loaded once, wait in LDS for the output pass.  Each thread reads back only
  // the runs it wrote, so the LDS serves as per-thread storage: no barrier, and 16 consecutive
  // bytes per lane read conflict-free.
  __shared__ Raw8<BF16> gb[2][NCH * THREADS];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t col = (int64_t)(c * THREADS + tid) * 8;
    Raw8<BF16> g{}, b{};
    if (ln && in(c)) {
      g = load_raw8<BF16>(r.gamma, col);
      if (has_beta) b = load_raw8<BF16>(r.beta, col);
    }
    gb[0][c * THREADS + tid] = g;
    gb[1][c * THREADS + tid] = b;
  }
  auto load_row = [&](int64_t row, Raw8<BF16>(&x)[NCH]) __attribute__((always_inline)) {
    const bool ok = row < r.rows;
    const char* base = (const char*)r.residual + (ok ? row * H * ES : 0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, ok ? (int)(H * ES) : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (BF16) {
        x[c].u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[c], 0, 0));
      } else {
        x[c].a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[c], 0, 0));
        x[c].b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[c] + 16, 0, 0));
      }
    }
  };
  // A fresh copy of a raw run for each pass: the compiler may not keep the unpacked fp32 values
  // of one pass for the next (that would double the row's registers).
  auto fresh = [](Raw8<BF16> q) __attribute__((always_inline)) {
    if constexpr (BF16) {
      asm volatile("" : "+v"(q.u.x), "+v"(q.u.y), "+v"(q.u.z), "+v"(q.u.w));
    } else {
      asm volatile("" : "+v"(q.a), "+v"(q.b));
    }
    return q;
  };
  auto process = [&](int64_t row, const Raw8<BF16>(&x)[NCH]) __attribute__((always_inline)) {
    const int64_t ooff = row * (r.ld_out > 0 ? r.ld_out : H);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float v[8];
      unpack8<BF16>(fresh(x[c]), v);
      if (has_h && in(c)) {
        F8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = v[e];
        store8<BF16>(r.h_out, ooff + (int64_t)(c * THREADS + tid) * 8, o);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) sum += v[e] + v[e + 1];
    }
    if (!ln) return;
    const float inv_h = 1.0f / (float)H;
    const float mean = block_sum<THREADS>(sum, red) * inv_h;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (in(c)) {
        float v[8];
        unpack8<BF16>(fresh(x[c]), v);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float a0 = v[e] - mean, a1 = v[e + 1] - mean;
          sq += a0 * a0 + a1 * a1;
        }
      }
    }
    const float var = block_sum<THREADS>(sq, red) * inv_h;
    const float rstd = 1.0f / sqrtf(var + r.eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (in(c)) {
        float v[8], gv[8], bv[8];
        unpack8<BF16>(fresh(x[c]), v);
        unpack8<BF16>(gb[0][c * THREADS + tid], gv);
        unpack8<BF16>(gb[1][c * THREADS + tid], bv);
        F8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y.v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
        store8<BF16>(r.y_out, ooff + (int64_t)(c * THREADS + tid) * 8, y);
      }
    }
  };
  // Rows are prefetched two ahead through three rotating buffers: the wait for a row's loads
  // also covers every older access of the workgroup, and two rows back the stores have long
  // completed, so that wait is not held up by the previous row's stores.
  const int64_t step = gridDim.x;
  Raw8<BF16> xa[NCH], xb[NCH], xc[NCH];
  load_row(blockIdx.x, xa);
  load_row(blockIdx.x + step, xb);
  for (int64_t row = blockIdx.x; row < r.rows; row += 3 * step) {
    load_row(row + 2 * step, xc);
    __builtin_amdgcn_sched_barrier(0);
    process(row, xa);
    if (row + step >= r.rows) break;
    load_row(row + 3 * step, xa);
    __builtin_amdgcn_sched_barrier(0);
    process(row + step, xb);
    if (row + 2 * step >= r.rows) break;
    load_row(row + 4 * step, xb);
    __builtin_amdgcn_sched_barrier(0);
    process(row + 2 * step, xc);
  }
}

// Workgroups of one kernel instance resident per compute unit, queried once per process
// (the first call on any device answers for all: every device here is the same gfx950).
template <class K>
int resident_per_cu(K kernel, int threads) {
  static std::atomic<int> n{0};
  int v = n.load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 1;
    }
    n.store(v, std::memory_order_relaxed);
  }
  return v;
}

// Rows per launch: a workgroup loops over rows blockIdx.x, + gridDim.x, ...  With partials
// to sum, up to 16 workgroups per compute unit (two rows each for the 8192-row block
// reduces: 5.72 vs 5.58 TB/s for one row per workgroup on MI355X).  Without partials, as many
// workgroups as are resident at once, each prefetching its next rows (ln_rows_kernel, for bf16
// rows of up to 16384 elements: its row buffers fit the registers and gamma and beta 64 KB of LDS).
template <int THREADS, int NCH, bool BF16, bool FULL>
hipError_t launch_variant(const ReduceDesc& r, hipStream_t stream) {
  const int cus = device_cus();
  if constexpr (BF16 && NCH * THREADS <= 2048) {
    if (r.n_parts == 0) {
      auto k = ln_rows_kernel<THREADS, NCH, BF16, FULL>;
      const int64_t blocks = min(r.rows, (int64_t)resident_per_cu(k, THREADS) * cus);
      hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(THREADS), 0, stream, r);
      return hipGetLastError();
    }
  }
  const int64_t blocks = min(r.rows, (int64_t)16 * cus);
  const dim3 grid((unsigned)blocks), block(THREADS);
  const bool parts = r.n_parts > 0, res = r.residual != nullptr, ln = r.gamma != nullptr;
  if constexpr (BF16) {
    if (parts && r.parts_bf16) {
#define TPK_REDUCE_LAUNCH_PB(R, L) \
  hipLaunchKernelGGL((reduce_ln_kernel<THREADS, NCH, true, FULL, true, R, L, true>), grid, block, 0, stream, r)
      if (res && ln) TPK_REDUCE_LAUNCH_PB(true, true);
      else if (res) TPK_REDUCE_LAUNCH_PB(true, false);
      else if (ln) TPK_REDUCE_LAUNCH_PB(false, true);
      else TPK_REDUCE_LAUNCH_PB(false, false);
#undef TPK_REDUCE_LAUNCH_PB
      return hipGetLastError();
    }
  }
  if (r.parts_bf16 && parts) return hipErrorInvalidValue;  // bf16 partials need bf16 io
#define TPK_REDUCE_LAUNCH(P, R, L) \
  hipLaunchKernelGGL((reduce_ln_kernel<THREADS, NCH, BF16, FULL, P, R, L>), grid, block, 0, stream, r)
  if (parts && res && ln) TPK_REDUCE_LAUNCH(true, true, true);
  else if (parts && res) TPK_REDUCE_LAUNCH(true, true, false);
  else if (parts && ln) TPK_REDUCE_LAUNCH(true, false, true);
  else if (parts) TPK_REDUCE_LAUNCH(true, false, false);
  else if (ln) TPK_REDUCE_LAUNCH(false, true, true);  // no partials: the residual is required
  else TPK_REDUCE_LAUNCH(false, true, false);
#undef TPK_REDUCE_LAUNCH
  return hipGetLastError();
}

template <int THREADS, int NCH>
hipError_t launch_t(const ReduceDesc& r, hipStream_t stream) {
  const bool full = r.H == (int64_t)NCH * THREADS * 8;
  if (r.bf16) return full ? launch_variant<THREADS, NCH, true, true>(r, stream)
                          : launch_variant<THREADS, NCH, true, false>(r, stream);
  return full ? launch_variant<THREADS, NCH, false, true>(r, stream)
              : launch_variant<THREADS, NCH, false, false>(r, stream);
}

}  // namespace

hipError_t launch_reduce_ln(const ReduceDesc& r, hipStream_t stream) {
  if (r.rows <= 0) return hipSuccess;
  if (r.rows > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t runs = (r.H + 7) / 8;  // runs of 8 elements per row
  if (runs <= 64 * 1) return launch_t<64, 1>(r, stream);
  if (runs <= 128 * 1) return launch_t<128, 1>(r, stream);
  if (runs <= 256 * 1) return launch_t<256, 1>(r, stream);
  if (runs <= 256 * 2) return launch_t<256, 2>(r, stream);
  if (runs <= 256 * 3) return launch_t<256, 3>(r, stream);
  if (runs <= 256 * 4) return launch_t<256, 4>(r, stream);
  if (runs <= 256 * 6) return launch_t<256, 6>(r, stream);
  if (runs <= 256 * 8) return launch_t<256, 8>(r, stream);
  if (runs <= 512 * 6) return launch_t<512, 6>(r, stream);
  if (runs <= 512 * 8) return launch_t<512, 8>(r, stream);
  if (runs <= 1024 * 8) return launch_t<1024, 8>(r, stream);
  return hipErrorInvalidValue;
}

}  // namespace tpk
