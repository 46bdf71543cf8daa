// Per-head softmax attention over one rank's heads, gfx950, head_dim 128, bf16 in/out.
//
//   O_h = softmax(Q_h K_h^T / sqrt(d) + causal mask) V_h  for each sequence and head
//
// (0539edu.com TP tutorial section 1.2.2, formulas 1.8-1.13: each head attends with its
// own Q, K, V, independently of the other heads, which is what lets the heads be split
// across ranks with no exchange -- pwwt.cn section 2.2, figure 4.)
//
// One workgroup = 128 queries of one (sequence, head), 4 waves of 32 queries each, two
// workgroups per compute unit, so two waves per SIMD.  Keys stream through LDS in blocks of 64
// with the online (running-max) softmax, so the S x S score matrix never exists.  The K and V
// blocks go HBM -> LDS directly (buffer loads into LDS: no register round trip, no LDS store
// instructions), each wave fetching 16 of the 64 rows, one block ahead of their use.  The
// products are computed transposed so that every softmax row lives inside one lane pair:
//   S^T[key, query] = K Q^T   -- v_mfma_f32_32x32x16_bf16, A = K rows from LDS (16-byte
//                               reads), B = the wave's Q fragments held in registers;
//                               lane l owns query l % 32 and 16 keys per 32-key half, so
//                               the row max / sum need one exchange with lane l ^ 32
//                               (v_permlane32_swap).
//   O^T[d, query] += V^T P^T -- A = V^T fragments read from the row-major V block with the
//                               gfx950 LDS transpose read (ds_read_b64_tr_b16), B = P^T
//                               taken straight from the S^T accumulators converted to bf16
//                               (the key order inside a fragment is the accumulator's
//                               order, used identically for A and B).
// Software pipeline: iteration j computes block j+1's scores while block j's softmax runs,
// its work cut into short items placed one after each score MFMA, and then block j's PV
// product.  A wave cannot hide a long run of its own vector-ALU work behind its MFMAs, but
// with short items between the MFMAs and two waves per SIMD, each wave's items issue while
// the other's MFMAs run.
// LDS arrangement (no bank conflicts by construction; the LDS serves 16-byte reads 16 lanes
// at a time from 64 four-byte banks, and 8-byte transpose reads 32 lanes at a time):
//   K block: 64 rows (keys) x 256 bytes, 16-byte chunk c of row r at chunk c ^ (r & 15): the
//            16 rows of a read group hit 16 distinct chunk positions.
//   V block: 64 rows x 256 bytes, chunk c of row r at chunk c ^ 4 (r & 3): a transpose read
//            covers 4 consecutive rows x 32 bytes per 16 lanes, and the 8 (row, 32-byte pair)
//            positions of 32 lanes land on 8 distinct bank ranges.
// The arrangement is set by which global chunk each lane fetches, since an LDS-direct load
// writes lane i's 16 bytes at 16 i.
// Every wave runs every key block of its workgroup (a block above a wave's queries is fully
// masked and adds nothing), which keeps the barriers uniform; workgroups are launched
// heaviest (last query block) first.  The output tile is staged through LDS for 16-byte
// stores.
#include "lds_dma.hpp"

namespace tpk {
namespace {

using dma::i32x4_t;
using dma::static_for;

constexpr int AQ = 128;             // queries per workgroup
constexpr int AK = 64;              // keys per block
constexpr int D = 128;              // head dim
constexpr int NT = 256;             // threads: 4 waves
constexpr int TILE = AK * D * 2;    // 16 KB: one K or V block
constexpr int OPITCH = 2 * D + 16;  // 272-byte rows of the output staging tile

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;

__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const char* p, int second_offset) {
  const lds_char_t* lp = (const lds_char_t*)p;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lp);
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lp + second_offset));
  i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& s, int r0) {
  uint4 u;
  u.x = pack_bf16x2(s[r0 + 0], s[r0 + 1]);
  u.y = pack_bf16x2(s[r0 + 2], s[r0 + 3]);
  u.z = pack_bf16x2(s[r0 + 4], s[r0 + 5]);
  u.w = pack_bf16x2(s[r0 + 6], s[r0 + 7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// v_permlane32_swap with both operands v: of its two results, one holds v of this lane and
// the other v of lane l ^ 32 (which is which depends on the half), so the pair's max and sum
// are the lane pair's max and sum in every lane.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnDesc a) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K buffers 0, 1; V 0, 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, i32 = lane & 31;
  const int64_t seq = a.seq;
  const int seqi = (int)seq;
  const int hl = a.hl;
  const int nqb = (int)((seq + AQ - 1) / AQ);
  const int hb = hl * (int)a.batch;
  const int qb = nqb - 1 - (int)(blockIdx.x / hb);
  const int rest = (int)(blockIdx.x % hb);
  const int head = rest % hl;
  const int64_t bt = rest / hl;

  const int64_t ld = 3LL * hl * D;  // elements per token row of [Q | K | V]
  const bf16_t* base = a.qkv + bt * seq * ld;
  const bf16_t* Qg = base + (int64_t)head * D;
  const bf16_t* Kg = base + (int64_t)hl * D + (int64_t)head * D;
  const bf16_t* Vg = base + 2LL * hl * D + (int64_t)head * D;
  const bool causal = a.causal != 0;

  const int q0 = qb * AQ;
  const int qw = q0 + 32 * w;        // first query of this wave
  const int mq = qw + i32;           // this lane's query

  // ---- LDS-direct loads of key block kb into buffer buf: this wave fills rows
  // 16 w + 4 i + lane / 16 (i < 4) of the K and V tiles, physical chunk lane % 16, fetching
  // the logical chunk that belongs there.  One buffer resource per tile spans the wave's 16
  // rows (fewer at the end of the sequence, none past it), so rows outside read as zeros;
  // seq < 2^30 and a row is under 2^24 bytes, so the offsets fit 32 bits.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t*)smem;
  const uint32_t ldb = (uint32_t)(ld * 2);  // bytes per token row
  const int lr = lane >> 4, pch = lane & 15;
  uint32_t kofs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    kofs[i] = (uint32_t)(lr + 4 * i) * ldb + (uint32_t)((pch ^ (4 * i + lr)) << 4);
  const uint32_t vofs = (uint32_t)lr * ldb + (uint32_t)((pch ^ (4 * lr)) << 4);
  auto rows_rsrc = [&](const bf16_t* src, int kb) __attribute__((always_inline)) {
    const int row0 = kb * AK + 16 * w;
    const int n = min(max(seqi - row0, 0), 16);
    return dma::rsrc(src + (int64_t)row0 * ld, (uint32_t)n * ldb);
  };
  auto load_block_k = [&](int kb, int buf) __attribute__((always_inline)) {
    const i32x4_t rk = rows_rsrc(Kg, kb);
    const uint32_t kl = lds0 + (uint32_t)(buf * TILE + w * 4096);
    static_for<4>([&](auto IC) {
      constexpr int I = decltype(IC)::value;
      dma::load16<I * 1024>(kl, kofs[I], rk, 0u);
    });
  };
  auto load_block_v = [&](int kb, int buf) __attribute__((always_inline)) {
    const i32x4_t rv = rows_rsrc(Vg, kb);
    const uint32_t vl = lds0 + (uint32_t)((2 + buf) * TILE + w * 4096);
    static_for<4>([&](auto IC) {
      constexpr int I = decltype(IC)::value;
      dma::load16<I * 1024>(vl, vofs + (uint32_t)(4 * I) * ldb, rv, 0u);
    });
  };

  // ---- fragment addresses (bytes within a tile)
  //   K fragment (jb, s): key row 32 jb + lane % 32, d 16 s + 8 h .. +7, logical chunk
  //   2 s + h at (2 s + h) ^ (row & 15) = 2 s ^ (h ^ (lane & 15)) since 2 s has bit 0 clear.
  const int krow = i32 * 256, kxr = h ^ (i32 & 15);
  //   V^T fragment (u, db): lane (16 G + q + 4 s') of group G addresses key row 16 u + 4 h + s'
  //   (second read: + 8 rows), d 32 db + 16 (G & 1) + 4 q .. +3.
  const int G = lane >> 4, li = lane & 15, vq = li & 3, vs = li >> 2;
  int vrd[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vrd[db] = (4 * h + vs) * 256 + ((4 * (db ^ vs) + 2 * (G & 1) + (vq >> 1)) << 4) + 8 * (vq & 1);

  // ---- Q^T as the MFMA B operand: lane (query mq, half h) holds Q[mq][16 s + 8 h .. + 8].
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (mq < seq) v = *(const uint4*)(Qg + (int64_t)mq * ld + 16 * s + 8 * h);
    qf[s] = __builtin_bit_cast(bf16x8_t, v);
  }

  const int64_t kend = causal ? min(seq, (int64_t)q0 + AQ) : seq;
  const int nkb = (int)((kend + AK - 1) / AK);
  const float scale = a.scale_log2;

  // ---- state.  S[b][jb]: scores S^T of keys 32 jb .. +31 of a block for the wave's 32
  // queries; two blocks in flight (b), so block j+1's scores are computed while block j's
  // softmax runs.  O^T blocks db (d 32 db .. +31).
  f32x16_t S[2][2];
  f32x16_t O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[db][r] = 0.0f;
  float m_run = -INFINITY;  // running offset of this lane's query (log2 units)
  float l_run = 0.0f;       // running sum over this lane half's keys
  float m_use = 0.0f, alpha = 1.0f, mx = -INFINITY, psum = 0.0f;
  bool moved = false;
  bf16x8_t pf[4];  // P^T fragments u (keys 16 u .. +15 of the block) of the current block

  // Score MFMA m (0..15) of a block: key half jb = m % 2, d-step ss = m / 2 (the two chains
  // alternate, so consecutive MFMAs are independent).  Its K fragment is read two MFMAs ahead
  // into a ring of three.
  bf16x8_t kf[3];
  auto read_k = [&](const char* kt, int m) __attribute__((always_inline)) {
    kf[m % 3] = *(const bf16x8_t*)(kt + (m % 2) * 32 * 256 + krow + ((2 * (m / 2) ^ kxr) << 4));
  };
  // PV MFMA m (0..15): key step u = m / 4, d block db = m % 4; V^T fragment read likewise.
  bf16x8_t vf[3];
  auto read_v = [&](const char* vt, int m) __attribute__((always_inline)) {
    vf[m % 3] = ds_read_tr_pair(vt + (m / 4) * 16 * 256 + vrd[m % 4], 8 * 256);
  };

  // Softmax work items of a block, in order, each a few ALU instructions, placed one after
  // each MFMA (a wave issues in order, so an item longer than an MFMA would hold back the next
  // one, and two waves per SIMD fill each other's gaps):
  //   0-3    row max over values 8 (t % 2) .. +7 of key half t / 2
  //   4      the lane-pair exchange and the new offset
  //   5-12   exponentials: key half (t - 5) / 4, values 4 ((t - 5) % 4) .. +3
  //   13-16  the bf16 P^T fragment u = t - 13 and its sum
  // The lazy offset moves only when the block's max exceeds it by more than 8 (log2 units):
  // the probabilities stay below 2^8 and the output rescale is skipped unless some lane of
  // the wave moved; the final division uses a sum taken with the same offsets, so the result
  // is unchanged.  The sum is taken over the bf16 probabilities the PV product uses.  Each
  // item ends by pinning its results (an empty asm statement that takes them as operands):
  // the items are pure arithmetic, which the compiler would otherwise sink next to their
  // first use and out of the MFMA shadow they are placed in.
  auto item = [&](f32x16_t (&Sc)[2], auto TC) __attribute__((always_inline)) {
    constexpr int t = decltype(TC)::value;
    if constexpr (t < 4) {
      constexpr int jb = t / 2, r0 = 8 * (t % 2);
      float m = fmaxf(fmaxf(Sc[jb][r0], Sc[jb][r0 + 1]), Sc[jb][r0 + 2]);
      m = fmaxf(fmaxf(m, Sc[jb][r0 + 3]), Sc[jb][r0 + 4]);
      m = fmaxf(fmaxf(m, Sc[jb][r0 + 5]), Sc[jb][r0 + 6]);
      m = fmaxf(m, Sc[jb][r0 + 7]);
      mx = t == 0 ? m : fmaxf(mx, m);
      asm volatile("" : "+v"(mx));
    } else if constexpr (t == 4) {
      const float bm = pair_max(mx) * scale;  // scale > 0
      moved = bm > m_run + 8.0f;
      const float m_new = moved ? bm : m_run;
      alpha = moved ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      // a row with every key masked so far keeps offset -inf; its probabilities are 0
      m_use = m_new == -INFINITY ? 0.0f : m_new;
      asm volatile("" : "+v"(m_use), "+v"(alpha));
    } else if constexpr (t < 13) {
      constexpr int e = t - 5, jb = e / 4, r0 = 4 * (e % 4);
#pragma unroll
      for (int r = r0; r < r0 + 4; ++r) {
        Sc[jb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[jb][r], scale, -m_use));
        asm volatile("" : "+v"(Sc[jb][r]));
      }
    } else {
      constexpr int u = t - 13;
      pf[u] = pack8(Sc[u >> 1], 8 * (u & 1));
      const uint4 wv = __builtin_bit_cast(uint4, pf[u]);
      const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
      float ps = u == 0 ? 0.0f : psum;
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv.x), one, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv.y), one, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv.z), one, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv.w), one, ps, false);
      psum = ps;
      asm volatile("" : "+v"(pf[u]), "+v"(psum));
    }
  };

  // Score MFMAs of one block into Sn from K tile kt, with extra(m) after MFMA m.
  auto scores = [&](f32x16_t (&Sn)[2], const char* kt, auto&& extra) __attribute__((always_inline)) {
    read_k(kt, 0);
    read_k(kt, 1);
    static_for<16>([&](auto MC) {
      constexpr int m = decltype(MC)::value;
      constexpr int jb = m % 2, ss = m / 2;
      const f32x16_t zero = {};
      Sn[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m % 3], qf[ss], ss == 0 ? zero : Sn[jb],
                                                       0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m + 2 < 16) read_k(kt, m + 2);
      extra(MC);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // PV MFMAs of one block from V tile vt, with extra(m) after MFMA m.
  auto pv = [&](const char* vt, auto&& extra) __attribute__((always_inline)) {
    read_v(vt, 0);
    read_v(vt, 1);
    static_for<16>([&](auto MC) {
      constexpr int m = decltype(MC)::value;
      constexpr int u = m / 4, db = m % 4;
      O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[m % 3], pf[u], O[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m + 2 < 16) read_v(vt, m + 2);
      extra(MC);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  const char* const kt0 = smem;             // K buffer 0 (buffer 1: + TILE)
  const char* const vt0 = smem + 2 * TILE;  // V buffer 0 (buffer 1: + TILE)

  // Iteration t (P = t % 2): block t's softmax and PV product, and block t+1's scores (NEXT).
  // Before it, every wave's loads of K block t+1 and V block t (issued one iteration earlier)
  // have landed and every wave is done with iteration t-1, whose K block t and V block t-1
  // buffers take the loads of K block t+2 and V block t+1.
  auto iteration = [&](auto PC, auto NEXTC, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(PC)::value;
    constexpr bool NEXT = decltype(NEXTC)::value;
    dma::wait_vmcnt<0>();
    dma::barrier();
    if (t + 2 < nkb) load_block_k(t + 2, P);
    if (t + 1 < nkb) load_block_v(t + 1, 1 - P);
    const int j0 = t * AK;
    if ((causal && j0 + AK - 1 > qw) || j0 + AK > seq) {  // wave-uniform
      // key = j0 + 32 jb + 8 (r / 4) + 4 h + r % 4 is visible iff it is <= klim + j0 + 4 h
      const int klim = (causal ? min(mq, seqi - 1) : seqi - 1) - j0 - 4 * h;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[P][jb][r] = (32 * jb + 8 * (r >> 2) + (r & 3)) <= klim ? S[P][jb][r] : -INFINITY;
    }
    if constexpr (NEXT) {
      scores(S[1 - P], kt0 + (1 - P) * TILE, [&](auto MC) {
        constexpr int m = decltype(MC)::value;
        item(S[P], std::integral_constant<int, m>{});  // items 0-15
      });
    } else {
      static_for<16>([&](auto IC) { item(S[P], IC); });
    }
    // O rescale when some lane's offset moved (rare: the lazy offset), before this block's
    // products are added.
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    pv(vt0 + P * TILE, [&](auto MC) {
      constexpr int m = decltype(MC)::value;
      if constexpr (m == 0) item(S[P], std::integral_constant<int, 16>{});
    });
    l_run = l_run * alpha + psum;
  };

  // ---- prologue: K blocks 0 and 1 and V block 0; the scores of block 0
  load_block_k(0, 0);
  load_block_v(0, 0);
  if (nkb > 1) load_block_k(1, 1);
  dma::wait_vmcnt<0>();
  dma::barrier();
  scores(S[0], kt0, [](auto) {});
  using std::integral_constant;
  int t = 0;
  for (; t + 2 < nkb; t += 2) {
    iteration(integral_constant<int, 0>{}, integral_constant<bool, true>{}, t);
    iteration(integral_constant<int, 1>{}, integral_constant<bool, true>{}, t + 1);
  }
  if (nkb - t == 2) {
    iteration(integral_constant<int, 0>{}, integral_constant<bool, true>{}, t);
    iteration(integral_constant<int, 1>{}, integral_constant<bool, false>{}, t + 1);
  } else {
    iteration(integral_constant<int, 0>{}, integral_constant<bool, false>{}, t);
  }

  // Normalise and stage O (row = query, 128 d) through LDS, reusing the tiles once every
  // wave is done with them.
  const float l_tot = pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  dma::barrier();
  char* os = smem + w * 32 * OPITCH;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = 32 * db + 8 * ii + 4 * h;
      uint2 pk;
      pk.x = pack_bf16x2(O[db][4 * ii + 0] * inv, O[db][4 * ii + 1] * inv);
      pk.y = pack_bf16x2(O[db][4 * ii + 2] * inv, O[db][4 * ii + 3] * inv);
      *(uint2*)(os + i32 * OPITCH + 2 * d0) = pk;
    }
  __syncthreads();
  const int64_t ldo = (int64_t)hl * D;
  bf16_t* og = a.out + bt * seq * ldo + (int64_t)head * D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i;
    const int row = c >> 4, dc = (c & 15) * 8;
    const int64_t q = qw + row;
    if (q < seq) *(uint4*)(og + q * ldo + dc) = *(const uint4*)(os + row * OPITCH + 2 * dc);
  }
}

}  // namespace

hipError_t launch_attention(const AttnDesc& a, hipStream_t stream) {
  if (a.d != D) return hipErrorInvalidValue;
  if (a.seq > 0x3fffffff) return hipErrorInvalidValue;
  const int64_t nqb = (a.seq + AQ - 1) / AQ;
  const int64_t blocks = nqb * a.hl * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpk
