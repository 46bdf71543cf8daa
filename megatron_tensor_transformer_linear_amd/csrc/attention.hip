// Per-head softmax attention over one rank's heads, gfx950, head_dim 128, bf16 in/out.
//
//   O_h = softmax(Q_h K_h^T / sqrt(d) + causal mask) V_h  for each sequence and head
//
// (0539edu.com TP tutorial section 1.2.2, formulas 1.8-1.13: each head attends with its
// own Q, K, V, independently of the other heads, which is what lets the heads be split
// across ranks with no exchange -- pwwt.cn section 2.2, figure 4.)
//
// One workgroup = 128 queries of one (sequence, head), 4 waves of 32 queries each; keys
// stream through LDS in blocks of 64, double-buffered, with the online (running-max)
// softmax so the S x S score matrix never exists.  The products are computed transposed so
// that every softmax row lives inside one lane pair:
//   S^T[key, query] = K Q^T   -- v_mfma_f32_32x32x16_bf16, A = K rows from LDS (16-byte
//                               reads), B = the wave's Q fragments held in registers;
//                               lane l owns query l % 32 and 16 keys per 32-key block, so
//                               the row max / sum need one exchange with lane l ^ 32.
//   O^T[d, query] += V^T P^T -- A = V^T fragments read from the row-major V tile with the
//                               gfx950 LDS transpose read (ds_read_b64_tr_b16), B = P^T
//                               taken straight from the S^T accumulators converted to bf16
//                               (the key order inside a fragment is the accumulator's
//                               order, used identically for A and B).
// Causal work is skipped per wave above the diagonal; workgroups are launched heaviest
// (last query block) first.  The output tile is staged through LDS for 16-byte stores.
#include "common.hpp"

namespace tpk {
namespace {

constexpr int AQ = 128;  // queries per workgroup
constexpr int AK = 64;   // keys per block
constexpr int D = 128;   // head dim
constexpr int K_PITCH = D + 8;   // 272 B rows: 16-byte reads of 8 consecutive rows hit distinct banks
constexpr int V_PITCH = D + 16;  // 288 B rows: the 4 rows of one transpose read hit distinct banks
constexpr int NT = 256;

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

__device__ __forceinline__ bf16x8_t pack8(float a0, float a1, float a2, float a3, float a4,
                                          float a5, float a6, float a7) {
  uint4 u;
  u.x = pack_bf16x2(a0, a1);
  u.y = pack_bf16x2(a2, a3);
  u.z = pack_bf16x2(a4, a5);
  u.w = pack_bf16x2(a6, a7);
  return __builtin_bit_cast(bf16x8_t, u);
}

__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnDesc a) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2 * AK * K_PITCH];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2 * AK * V_PITCH];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5;
  const int64_t seq = a.seq;
  const int hl = a.hl;
  const int nqb = (int)((seq + AQ - 1) / AQ);
  const int hb = hl * (int)a.batch;
  const int qb = nqb - 1 - (int)(blockIdx.x / hb);
  const int rest = (int)(blockIdx.x % hb);
  const int head = rest % hl;
  const int64_t bt = rest / hl;

  const int64_t ld = 3LL * hl * D;
  const bf16_t* base = a.qkv + bt * seq * ld;
  const bf16_t* Qg = base + (int64_t)head * D;
  const bf16_t* Kg = base + (int64_t)hl * D + (int64_t)head * D;
  const bf16_t* Vg = base + 2LL * hl * D + (int64_t)head * D;

  const int q0 = qb * AQ;
  const int qw = q0 + 32 * w;        // first query of this wave
  const int mq = qw + (lane & 31);   // this lane's query

  // Q^T as the MFMA B operand: lane (query mq, half h) holds Q[mq][16 s + 8 h .. + 8].
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (mq < seq) v = *(const uint4*)(Qg + (int64_t)mq * ld + 16 * s + 8 * h);
    qf[s] = __builtin_bit_cast(bf16x8_t, v);
  }

  const int64_t kend = a.causal ? min(seq, (int64_t)q0 + AQ) : seq;
  const int nkb = (int)((kend + AK - 1) / AK);

  // K / V block staging: thread -> rows tid/16 + 16 i, 16-byte chunk (tid % 16).
  const int ld_row = tid >> 4, ld_dc = (tid & 15) * 8;
  uint4 rk[4], rv[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = (int64_t)kb * AK + ld_row + 16 * i;
      const bool ok = row < seq;
      rk[i] = ok ? *(const uint4*)(Kg + row * ld + ld_dc) : make_uint4(0, 0, 0, 0);
      rv[i] = ok ? *(const uint4*)(Vg + row * ld + ld_dc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)(Ks + buf * AK * K_PITCH + (ld_row + 16 * i) * K_PITCH + ld_dc) = rk[i];
      *(uint4*)(Vs + buf * AK * V_PITCH + (ld_row + 16 * i) * V_PITCH + ld_dc) = rv[i];
    }
  };

  float m_run = -INFINITY;  // running max of this lane's query (log2 domain)
  float l_run = 0.0f;       // running sum over this lane half's keys
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

  const int grp = lane >> 4, li = lane & 15;
  const int v_row = 4 * (grp >> 1) + (li >> 2);
  const int v_col = 16 * (grp & 1) + 4 * (li & 3);
  const float scale = a.scale_log2;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const int j0 = kb * AK;
    const bool active = !a.causal || j0 <= qw + 31;
    if (active) {
      const bf16_t* ks = Ks + cur * AK * K_PITCH;
      const bf16_t* vs = Vs + cur * AK * V_PITCH;
      f32x16_t s[2];
      const f32x16_t zero16 = {};
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int ss = 0; ss < 8; ++ss) {
          const bf16x8_t kf = *(const bf16x8_t*)(ks + (32 * jb + (lane & 31)) * K_PITCH + 16 * ss + 8 * h);
          s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ss], ss == 0 ? zero16 : s[jb], 0, 0, 0);
        }
      }
      // Mask, block max of the raw scores.  Element r of block jb is key
      // j0 + 32 jb + 8 (r / 4) + 4 h + r % 4 for query mq.  Every active block holds a key
      // <= the wave's first query (blocks are 64-aligned, waves 32-aligned), so no lane's
      // block is fully masked and its max is finite.
      const bool need_mask = (a.causal && j0 + AK - 1 > qw) || (j0 + AK > seq);
      if (need_mask) {  // wave-uniform: only diagonal and ragged-end blocks
        // key = j0 + kofs(jb, r) is visible iff key <= klim (branch-free selects)
        const int klim = (a.causal ? min(mq, (int)seq - 1) : (int)seq - 1) - j0 - 4 * h;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[jb][r] = (32 * jb + 8 * (r >> 2) + (r & 3)) <= klim ? s[jb][r] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale;  // log2 domain (scale > 0)
      // Lazy running max: the offset m_run moves only when this block's max exceeds it by
      // more than LAZY (log2 units), so the probabilities stay below 2^LAZY, and the output
      // rescale is skipped unless some lane of the wave moved.  The final normalisation
      // divides by a sum taken with the same offsets, so the result is unchanged.
      constexpr float LAZY = 8.0f;
      const bool move = mx > m_run + LAZY;
      const float m_new = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where the offset stays
      m_run = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][r], scale, -m_new));
          s[jb][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }

      // P^T fragments: MFMA u covers keys 16 u + 4 h + {0..3, 8..11}, which are the
      // accumulator rows r/4 = 2 (u % 2) and 2 (u % 2) + 1 of block u / 2.
      bf16x8_t pf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jb = u >> 1, r0 = 8 * (u & 1);
        pf[u] = pack8(s[jb][r0 + 0], s[jb][r0 + 1], s[jb][r0 + 2], s[jb][r0 + 3],
                      s[jb][r0 + 4], s[jb][r0 + 5], s[jb][r0 + 6], s[jb][r0 + 7]);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8_t vf = ds_read_tr_pair(vs + (16 * u + v_row) * V_PITCH + 32 * db + v_col,
                                              8 * V_PITCH);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[u], o[db], 0, 0, 0);
        }
    }
    if (kb + 1 < nkb) sstore(cur ^ 1);
    __syncthreads();
  }

  // Normalise and stage O (row = query, 128 d) through LDS, reusing the K buffers.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  bf16_t* os = Ks + w * 32 * K_PITCH;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = 32 * db + 8 * ii + 4 * h;
      uint2 pk;
      pk.x = pack_bf16x2(o[db][4 * ii + 0] * inv, o[db][4 * ii + 1] * inv);
      pk.y = pack_bf16x2(o[db][4 * ii + 2] * inv, o[db][4 * ii + 3] * inv);
      *(uint2*)(os + (lane & 31) * K_PITCH + d0) = pk;
    }
  __syncthreads();
  const int64_t ldo = (int64_t)hl * D;
  bf16_t* og = a.out + bt * seq * ldo + (int64_t)head * D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i;
    const int row = c >> 4, dc = (c & 15) * 8;
    const int64_t q = qw + row;
    if (q < seq) *(uint4*)(og + q * ldo + dc) = *(const uint4*)(os + row * K_PITCH + dc);
  }
}

}  // namespace

hipError_t launch_attention(const AttnDesc& a, hipStream_t stream) {
  if (a.d != D) return hipErrorInvalidValue;
  const int64_t nqb = (a.seq + AQ - 1) / AQ;
  const int64_t blocks = nqb * a.hl * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpk
