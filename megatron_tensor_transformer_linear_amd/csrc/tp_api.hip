// C ABI of the tensor-parallel layer-shard library: argument validation, shard-offset
// arithmetic (64-bit integers) and kernel launches.  Every check runs before the first
// launch (the only earlier HIP calls query the device's compute-unit count), so an invalid
// call launches nothing and leaves its outputs untouched.
#include <math.h>

#include <mutex>

#include "../../include/tp_shard.h"
#include "common.hpp"

using namespace tpk;

// The library's own scratch for tp_attn_head_shard_noalloc, the entry point for callers that
// cannot allocate: one array per GPU, held from the module's load until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host it names a
// stand-in, not device memory); it uses the device address hipGetSymbolAddress returns for
// the current device (scratch_address below).
static __device__ __align__(256) char scratch[TP_ATTN_SCRATCH_BYTES];

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The GEMM tile addresses a 256-row panel of the activation operand and a 64-row panel of
// the weight with 32-bit byte offsets, which bounds the two leading dimensions.
constexpr int64_t MAX_LD_ACT = 1 << 21;
constexpr int64_t MAX_LD_WEIGHT = 1 << 23;
// The weight-gradient products contract over the sequence, which the tile counts in 32-bit.
constexpr int64_t MAX_SEQ_BWD = (int64_t)1 << 30;
// The attention kernel indexes the queries and keys of a sequence in 32 bits.
constexpr int64_t MAX_SEQ_ATTN = ((int64_t)1 << 30) - 1;
inline bool mult8(int64_t v) { return (v & 7) == 0; }

inline int check_rank(int rank, int world) {
  if (world < 1 || rank < 0 || rank >= world) return TP_ERR_RANK;
  return TP_OK;
}

inline int launched(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_LAUNCH; }

struct AttnSizes {
  int64_t T, hl, nb, qkv_bytes, a_bytes, split_bytes, total;
};

int attn_sizes(int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim, int world,
               AttnSizes* s) {
  if (world < 1) return TP_ERR_RANK;
  if (batch <= 0 || seq <= 0 || H <= 0 || n_heads <= 0 || head_dim <= 0) return TP_ERR_SHAPE;
  if ((int64_t)n_heads * head_dim != H || head_dim != 128) return TP_ERR_SHAPE;
  if (H > MAX_LD_ACT) return TP_ERR_SHAPE;
  // the attention kernel indexes queries in 32 bits and the projections tile the tokens in
  // 32 bits (both bounds hold before any product below is formed)
  if (seq > MAX_SEQ_ATTN || batch > INT32_MAX || batch * seq > INT32_MAX) return TP_ERR_SHAPE;
  if (n_heads % world) return TP_ERR_DIVISIBLE;
  s->T = batch * seq;
  s->hl = n_heads / world;
  s->nb = s->hl * head_dim;
  s->qkv_bytes = s->T * 3 * s->nb * 2;
  s->a_bytes = s->T * s->nb * 2;
  // fp32 partials of the QKV projection's narrow strip when its contraction is split (a
  // device query: the strip depends on the compute-unit count)
  s->split_bytes = gemm_bf16_split_workspace(s->T, 3 * s->nb, H);
  s->total = ((s->qkv_bytes + s->a_bytes + s->split_bytes) + 255) & ~(int64_t)255;
  return TP_OK;
}

// Rank `rank`'s row-parallel product into Z [seq, N]: fp32, written (EPI_PARTIAL_F32) or
// added to what Z holds (EPI_ACC_F32); or bf16, written (EPI_STORE, bf16 io only).
int row_linear(const void* X, int64_t ldx, const void* W, void* Z, int64_t seq, int64_t K,
               int64_t N, int rank, int world, int epi, int dtype, void* stream) {
  if (!X || !W || !Z) return TP_ERR_NULL;
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (seq <= 0 || K <= 0 || N <= 0) return TP_ERR_SHAPE;
  if (K % world) return TP_ERR_DIVISIBLE;
  const int64_t kl = K / world;
  if (ldx < kl) return TP_ERR_SHAPE;
  if (ldx > MAX_LD_ACT || N > MAX_LD_WEIGHT) return TP_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Z)) return TP_ERR_ALIGN;
  if (!mult8(ldx) || !mult8(kl) || !mult8(N)) return TP_ERR_ALIGN;

  const size_t es = dtype == TP_BF16 ? 2 : 4;
  GemmDesc g;
  g.A = X;                                             // the rank's input shard [seq, K/world]
  g.lda = ldx;
  g.B = (const char*)W + (size_t)rank * kl * N * es;   // row block `rank` of W[K, N]
  g.ldb = N;
  g.b_blk = N;
  g.b_blk_stride = 0;
  g.n_off = 0;
  g.C = Z;
  g.ldc = N;
  g.M = seq;
  g.N = N;
  g.K = kl;
  g.epi = epi;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  return launched(dtype == TP_BF16 ? launch_gemm_bf16(g, s) : launch_gemm_f32(g, s));
}

// Rank `rank`'s attention head shard; its output projection writes (EPI_PARTIAL_F32) or adds
// to (EPI_ACC_F32) the fp32 Z [batch*seq, H], or writes it in bf16 (EPI_STORE).
int attn_head_shard(const void* Xn, const void* Wqkv, const void* Wo, void* Zpart,
                    int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim, int rank,
                    int world, int causal, int epi, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!Xn || !Wqkv || !Wo || !Zpart) return TP_ERR_NULL;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  AttnSizes s;
  if (int st = attn_sizes(batch, seq, H, n_heads, head_dim, world, &s)) return st;
  if (!workspace || workspace_bytes < (size_t)s.total) return TP_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return TP_ERR_ALIGN;
  if (!aligned16(Xn) || !aligned16(Wqkv) || !aligned16(Wo) || !aligned16(Zpart))
    return TP_ERR_ALIGN;

  bf16_t* ws_qkv = (bf16_t*)workspace;
  bf16_t* ws_a = (bf16_t*)((char*)workspace + s.qkv_bytes);
  float* ws_split = s.split_bytes ? (float*)((char*)workspace + s.qkv_bytes + s.a_bytes) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();

  // Column-parallel QKV: logical column n of the rank's [Q_r | K_r | V_r] is physical column
  // (n / nb) * H + rank * nb + n % nb of [Wq | Wk | Wv].
  GemmDesc q;
  q.A = Xn;
  q.lda = H;
  q.B = (const bf16_t*)Wqkv + (size_t)rank * s.nb;
  q.ldb = 3 * H;
  q.b_blk = s.nb;
  q.b_blk_stride = H;
  q.n_off = 0;
  q.C = ws_qkv;
  q.ldc = 3 * s.nb;
  q.M = s.T;
  q.N = 3 * s.nb;
  q.K = H;
  q.epi = EPI_STORE;
  if (launch_gemm_bf16_split(q, ws_split, st) != hipSuccess) return TP_ERR_LAUNCH;

  AttnDesc a;
  a.qkv = ws_qkv;
  a.out = ws_a;
  a.batch = batch;
  a.seq = seq;
  a.hl = (int)s.hl;
  a.d = head_dim;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  if (launch_attention(a, st) != hipSuccess) return TP_ERR_LAUNCH;

  // Row-parallel output projection over the rank's rows of Wo.
  GemmDesc o;
  o.A = ws_a;
  o.lda = s.nb;
  o.B = (const bf16_t*)Wo + (size_t)rank * s.nb * H;
  o.ldb = H;
  o.b_blk = H;
  o.b_blk_stride = 0;
  o.n_off = 0;
  o.C = Zpart;
  o.ldc = H;
  o.M = s.T;
  o.N = H;
  o.K = s.nb;
  o.epi = epi;
  return launched(launch_gemm_bf16(o, st));
}

// Device address of `scratch` on the current device, looked up once per device (each GPU
// holds its own copy of the array at its own address).
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return TP_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return TP_ERR_LAUNCH;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "TP_OK: success";
    case TP_ERR_NULL: return "TP_ERR_NULL: a required pointer is NULL";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE: invalid or unsupported size or leading dimension";
    case TP_ERR_DIVISIBLE: return "TP_ERR_DIVISIBLE: split dimension not divisible by world";
    case TP_ERR_RANK: return "TP_ERR_RANK: world < 1 or rank outside [0, world)";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unknown or unsupported dtype or activation";
    case TP_ERR_ALIGN: return "TP_ERR_ALIGN: misaligned pointer, leading dimension or shard offset";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_LAUNCH: return "TP_ERR_LAUNCH: kernel launch failed";
    case TP_ERR_SCRATCH:
      return "TP_ERR_SCRATCH: the sizes need more than the library's static scratch "
             "(TP_ATTN_SCRATCH_BYTES per GPU)";
    default: return "unknown tp_status";
  }
}

int tp_col_linear_gelu(const void* X, const void* W, void* Y, int64_t ldy, int64_t seq,
                       int64_t H, int64_t N, int rank, int world, int act, int dtype,
                       void* stream) {
  if (!X || !W || !Y) return TP_ERR_NULL;
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
  if (act != TP_ACT_NONE && act != TP_ACT_GELU_TANH) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (seq <= 0 || H <= 0 || N <= 0) return TP_ERR_SHAPE;
  if (N % world) return TP_ERR_DIVISIBLE;
  const int64_t nl = N / world;
  if (ldy < nl) return TP_ERR_SHAPE;
  if (H > MAX_LD_ACT || N > MAX_LD_WEIGHT) return TP_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return TP_ERR_ALIGN;
  if (!mult8(H) || !mult8(N) || !mult8(nl) || !mult8(ldy)) return TP_ERR_ALIGN;

  const size_t es = dtype == TP_BF16 ? 2 : 4;
  GemmDesc g;
  g.A = X;
  g.lda = H;
  g.B = (const char*)W + (size_t)rank * nl * es;  // column block `rank` of W[H, N]
  g.ldb = N;
  g.b_blk = nl;
  g.b_blk_stride = 0;
  g.n_off = 0;
  g.C = Y;
  g.ldc = ldy;
  g.M = seq;
  g.N = nl;
  g.K = H;
  g.epi = act == TP_ACT_GELU_TANH ? EPI_GELU_TANH : EPI_STORE;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  return launched(dtype == TP_BF16 ? launch_gemm_bf16(g, s) : launch_gemm_f32(g, s));
}

int tp_row_linear_partial(const void* X, int64_t ldx, const void* W, float* Zpart, int64_t seq,
                          int64_t K, int64_t N, int rank, int world, int dtype, void* stream) {
  return row_linear(X, ldx, W, Zpart, seq, K, N, rank, world, EPI_PARTIAL_F32, dtype, stream);
}

int tp_row_linear_fold(const void* X, int64_t ldx, const void* W, float* Zsum, int64_t seq,
                       int64_t K, int64_t N, int rank, int world, int accumulate, int dtype,
                       void* stream) {
  return row_linear(X, ldx, W, Zsum, seq, K, N, rank, world,
                    accumulate ? EPI_ACC_F32 : EPI_PARTIAL_F32, dtype, stream);
}

int tp_row_linear_partial_bf16(const void* X, int64_t ldx, const void* W, void* Zpart,
                               int64_t seq, int64_t K, int64_t N, int rank, int world,
                               void* stream) {
  return row_linear(X, ldx, W, Zpart, seq, K, N, rank, world, EPI_STORE, TP_BF16, stream);
}

int tp_col_linear_gelu_save(const void* X, const void* W, void* Y, int64_t ldy, void* U,
                            int64_t ldu, int64_t seq, int64_t H, int64_t N, int rank, int world,
                            int dtype, void* stream) {
  if (!X || !W || !Y || !U) return TP_ERR_NULL;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (seq <= 0 || H <= 0 || N <= 0) return TP_ERR_SHAPE;
  if (N % world) return TP_ERR_DIVISIBLE;
  const int64_t nl = N / world;
  if (ldy < nl || ldu < nl) return TP_ERR_SHAPE;
  if (H > MAX_LD_ACT || N > MAX_LD_WEIGHT) return TP_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || !aligned16(U)) return TP_ERR_ALIGN;
  if (!mult8(H) || !mult8(N) || !mult8(nl) || !mult8(ldy) || !mult8(ldu)) return TP_ERR_ALIGN;

  GemmDesc g;
  g.A = X;
  g.lda = H;
  g.B = (const bf16_t*)W + (size_t)rank * nl;  // column block `rank` of W[H, N]
  g.ldb = N;
  g.b_blk = nl;
  g.b_blk_stride = 0;
  g.n_off = 0;
  g.C = Y;
  g.ldc = ldy;
  g.M = seq;
  g.N = nl;
  g.K = H;
  g.epi = EPI_GELU_SAVE;
  g.aux = U;
  g.ldaux = ldu;
  (void)hipGetLastError();
  return launched(launch_gemm_bf16(g, (hipStream_t)stream));
}

int tp_row_linear_backward(const void* dZ, const void* W, const void* Y, int64_t ldy,
                           const void* U, int64_t ldu, void* dY, int64_t ld_dy, float* dW,
                           int64_t ld_dw, int64_t seq, int64_t K, int64_t N, int rank, int world,
                           int act, int accumulate, int dtype, void* stream) {
  if (!dZ || !W || (!dY && !dW)) return TP_ERR_NULL;
  if (dW && !Y) return TP_ERR_NULL;
  if (dY && act == TP_ACT_GELU_TANH && !U) return TP_ERR_NULL;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (act != TP_ACT_NONE && act != TP_ACT_GELU_TANH) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (seq <= 0 || K <= 0 || N <= 0 || seq > MAX_SEQ_BWD) return TP_ERR_SHAPE;
  if (K % world) return TP_ERR_DIVISIBLE;
  const int64_t kl = K / world;
  const bool use_u = dY && act == TP_ACT_GELU_TANH;
  if ((dY && ld_dy < kl) || (use_u && ldu < kl) || (dW && (ldy < kl || ld_dw < N)))
    return TP_ERR_SHAPE;
  // dZ is the K-contiguous operand of dY = dZ . W_r^T and W_r^T the K-contiguous B^T; Y^T is
  // the M-contiguous operand of dW = Y^T . dZ.
  if (N > MAX_LD_ACT || (dW && ldy > MAX_LD_ACT)) return TP_ERR_SHAPE;
  const void* ptrs[] = {dZ, W, Y, U, dY, dW};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;
  if (!mult8(N) || !mult8(kl)) return TP_ERR_ALIGN;
  if ((dY && !mult8(ld_dy)) || (use_u && !mult8(ldu)) || (dW && (!mult8(ldy) || !mult8(ld_dw))))
    return TP_ERR_ALIGN;

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (dY) {  // dY[t, j] = act'(U[t, j]) * sum_n dZ[t, n] W[rank*kl + j, n]
    GemmDesc g;
    g.A = dZ;
    g.lda = N;
    g.B = (const bf16_t*)W + (size_t)rank * kl * N;  // row block `rank` of W, read as B^T
    g.ldb = N;
    g.b_blk = kl;
    g.b_blk_stride = 0;
    g.n_off = 0;
    g.C = dY;
    g.ldc = ld_dy;
    g.M = seq;
    g.N = kl;
    g.K = N;
    g.layout = LAY_NT;
    g.epi = use_u ? EPI_GELU_BWD : EPI_STORE;
    g.aux = use_u ? const_cast<void*>(U) : nullptr;
    g.ldaux = use_u ? ldu : 0;
    if (launch_gemm_bf16(g, st) != hipSuccess) return TP_ERR_LAUNCH;
  }
  if (dW) {  // dW[j, n] (+)= sum_t Y[t, j] dZ[t, n]
    GemmDesc g;
    g.A = Y;
    g.lda = ldy;
    g.B = dZ;
    g.ldb = N;
    g.b_blk = N;
    g.b_blk_stride = 0;
    g.n_off = 0;
    g.C = dW;
    g.ldc = ld_dw;
    g.M = kl;
    g.N = N;
    g.K = seq;
    g.layout = LAY_TN;
    g.epi = accumulate ? EPI_ACC_F32 : EPI_PARTIAL_F32;
    if (launch_gemm_bf16(g, st) != hipSuccess) return TP_ERR_LAUNCH;
  }
  return TP_OK;
}

}  // extern "C"

namespace {
// tp_col_linear_backward with the input-gradient partial stored in fp32 (EPI_PARTIAL_F32) or
// in bf16 (EPI_STORE).
int col_linear_backward(const void* X, const void* W, const void* dU, int64_t ldu,
                        void* dXpart, float* dW, int64_t ld_dw, int64_t seq, int64_t H,
                        int64_t N, int rank, int world, int accumulate, int dtype, int dx_epi,
                        void* stream) {
  if (!X || !W || !dU || (!dXpart && !dW)) return TP_ERR_NULL;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (seq <= 0 || H <= 0 || N <= 0 || seq > MAX_SEQ_BWD) return TP_ERR_SHAPE;
  if (N % world) return TP_ERR_DIVISIBLE;
  const int64_t nl = N / world;
  if (ldu < nl || (dW && ld_dw < nl)) return TP_ERR_SHAPE;
  // dU is the K-contiguous operand of dX = dU . W_r^T and W_r^T (rows of W) the K-contiguous
  // B^T; X^T is the M-contiguous operand of dW = X^T . dU.
  if (ldu > MAX_LD_ACT || N > MAX_LD_ACT || H > MAX_LD_ACT) return TP_ERR_SHAPE;
  const void* ptrs[] = {X, W, dU, dXpart, dW};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;
  if (!mult8(H) || !mult8(N) || !mult8(nl) || !mult8(ldu) || (dW && !mult8(ld_dw)))
    return TP_ERR_ALIGN;

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (dXpart) {  // dXpart[t, h] = sum_j dU[t, j] W[h, rank*nl + j]
    GemmDesc g;
    g.A = dU;
    g.lda = ldu;
    g.B = (const bf16_t*)W + (size_t)rank * nl;  // column block `rank` of W, read as B^T
    g.ldb = N;
    g.b_blk = H;
    g.b_blk_stride = 0;
    g.n_off = 0;
    g.C = dXpart;
    g.ldc = H;
    g.M = seq;
    g.N = H;
    g.K = nl;
    g.layout = LAY_NT;
    g.epi = dx_epi;
    if (launch_gemm_bf16(g, st) != hipSuccess) return TP_ERR_LAUNCH;
  }
  if (dW) {  // dW[h, j] (+)= sum_t X[t, h] dU[t, j]
    GemmDesc g;
    g.A = X;
    g.lda = H;
    g.B = dU;
    g.ldb = ldu;
    g.b_blk = nl;
    g.b_blk_stride = 0;
    g.n_off = 0;
    g.C = dW;
    g.ldc = ld_dw;
    g.M = H;
    g.N = nl;
    g.K = seq;
    g.layout = LAY_TN;
    g.epi = accumulate ? EPI_ACC_F32 : EPI_PARTIAL_F32;
    if (launch_gemm_bf16(g, st) != hipSuccess) return TP_ERR_LAUNCH;
  }
  return TP_OK;
}
}  // namespace

extern "C" {

int tp_col_linear_backward(const void* X, const void* W, const void* dU, int64_t ldu,
                           float* dXpart, float* dW, int64_t ld_dw, int64_t seq, int64_t H,
                           int64_t N, int rank, int world, int accumulate, int dtype,
                           void* stream) {
  return col_linear_backward(X, W, dU, ldu, dXpart, dW, ld_dw, seq, H, N, rank, world,
                             accumulate, dtype, EPI_PARTIAL_F32, stream);
}

int tp_col_linear_backward_bf16(const void* X, const void* W, const void* dU, int64_t ldu,
                                void* dXpart, float* dW, int64_t ld_dw, int64_t seq, int64_t H,
                                int64_t N, int rank, int world, int accumulate, void* stream) {
  return col_linear_backward(X, W, dU, ldu, dXpart, dW, ld_dw, seq, H, N, rank, world,
                             accumulate, TP_BF16, EPI_STORE, stream);
}

size_t tp_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t H, int n_heads,
                               int head_dim, int world, int dtype) {
  if (dtype != TP_BF16) return 0;
  AttnSizes s;
  if (attn_sizes(batch, seq, H, n_heads, head_dim, world, &s) != TP_OK) return 0;
  return (size_t)s.total;
}

int tp_attn_head_shard(const void* Xn, const void* Wqkv, const void* Wo, float* Zpart,
                       int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                       int rank, int world, int causal, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return attn_head_shard(Xn, Wqkv, Wo, Zpart, batch, seq, H, n_heads, head_dim, rank, world,
                         causal, EPI_PARTIAL_F32, dtype, workspace, workspace_bytes, stream);
}

int tp_attn_head_shard_fold(const void* Xn, const void* Wqkv, const void* Wo, float* Zsum,
                            int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                            int rank, int world, int causal, int accumulate, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attn_head_shard(Xn, Wqkv, Wo, Zsum, batch, seq, H, n_heads, head_dim, rank, world,
                         causal, accumulate ? EPI_ACC_F32 : EPI_PARTIAL_F32, dtype, workspace,
                         workspace_bytes, stream);
}

int tp_attn_head_shard_bf16(const void* Xn, const void* Wqkv, const void* Wo, void* Zpart,
                            int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                            int rank, int world, int causal, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return attn_head_shard(Xn, Wqkv, Wo, Zpart, batch, seq, H, n_heads, head_dim, rank, world,
                         causal, EPI_STORE, TP_BF16, workspace, workspace_bytes, stream);
}

int tp_attn_head_shard_noalloc(const void* Xn, const void* Wqkv, const void* Wo, float* Zpart,
                               int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                               int rank, int world, int causal, int dtype, void* stream) {
  // Every check of tp_attn_head_shard except the workspace's, then the size limit, all before
  // the scratch lookup (the first call on a device) and any launch.
  if (!Xn || !Wqkv || !Wo || !Zpart) return TP_ERR_NULL;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  AttnSizes s;
  if (int st = attn_sizes(batch, seq, H, n_heads, head_dim, world, &s)) return st;
  if ((uint64_t)s.total > (uint64_t)TP_ATTN_SCRATCH_BYTES) return TP_ERR_SCRATCH;
  if (!aligned16(Xn) || !aligned16(Wqkv) || !aligned16(Wo) || !aligned16(Zpart))
    return TP_ERR_ALIGN;
  void* ws = nullptr;
  if (int st = scratch_address(&ws)) return st;
  return attn_head_shard(Xn, Wqkv, Wo, Zpart, batch, seq, H, n_heads, head_dim, rank, world,
                         causal, EPI_PARTIAL_F32, dtype, ws, (size_t)TP_ATTN_SCRATCH_BYTES, stream);
}

int tp_partial_reduce_residual_ln(const float* parts, int n_parts, int64_t part_stride,
                                  const void* residual, const void* gamma, const void* beta,
                                  float eps, void* h_out, void* y_out, int64_t rows, int64_t H,
                                  int dtype, void* stream) {
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
  if (n_parts < 0) return TP_ERR_SHAPE;
  if (n_parts > 0 && !parts) return TP_ERR_NULL;
  if (n_parts == 0 && !residual) return TP_ERR_NULL;
  if (gamma && !y_out) return TP_ERR_NULL;
  if (!gamma && !h_out) return TP_ERR_NULL;
  if (rows <= 0 || rows > INT32_MAX || H <= 0 || H > 65536) return TP_ERR_SHAPE;
  if (!(eps >= 0.0f) || isinf(eps)) return TP_ERR_SHAPE;
  if (n_parts > 1 && part_stride < rows * H) return TP_ERR_SHAPE;
  if (!mult8(H)) return TP_ERR_ALIGN;
  if (n_parts > 1 && (part_stride & 3)) return TP_ERR_ALIGN;
  const void* ptrs[] = {parts, residual, gamma, beta, h_out, y_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;

  ReduceDesc r;
  r.parts = parts;
  r.n_parts = n_parts;
  r.part_stride = part_stride;
  r.residual = residual;
  r.gamma = gamma;
  r.beta = beta;
  r.eps = eps;
  r.h_out = h_out;
  r.y_out = gamma ? y_out : nullptr;
  r.rows = rows;
  r.H = H;
  r.bf16 = dtype == TP_BF16;
  (void)hipGetLastError();
  return launched(launch_reduce_ln(r, (hipStream_t)stream));
}

int tp_partial_reduce_residual_ln_bf16(const void* parts, int n_parts, int64_t part_stride,
                                       const void* residual, const void* gamma, const void* beta,
                                       float eps, void* h_out, void* y_out, int64_t rows,
                                       int64_t H, void* stream) {
  if (n_parts < 0) return TP_ERR_SHAPE;
  if (n_parts > 0 && !parts) return TP_ERR_NULL;
  if (n_parts == 0 && !residual) return TP_ERR_NULL;
  if (gamma && !y_out) return TP_ERR_NULL;
  if (!gamma && !h_out) return TP_ERR_NULL;
  if (rows <= 0 || rows > INT32_MAX || H <= 0 || H > 65536) return TP_ERR_SHAPE;
  if (!(eps >= 0.0f) || isinf(eps)) return TP_ERR_SHAPE;
  if (n_parts > 1 && part_stride < rows * H) return TP_ERR_SHAPE;
  if (!mult8(H)) return TP_ERR_ALIGN;
  if (n_parts > 1 && !mult8(part_stride)) return TP_ERR_ALIGN;
  const void* ptrs[] = {parts, residual, gamma, beta, h_out, y_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;

  ReduceDesc r;
  r.parts = (const float*)parts;  // read as bf16 (parts_bf16)
  r.n_parts = n_parts;
  r.part_stride = part_stride;
  r.residual = residual;
  r.gamma = gamma;
  r.beta = beta;
  r.eps = eps;
  r.h_out = h_out;
  r.y_out = gamma ? y_out : nullptr;
  r.rows = rows;
  r.H = H;
  r.bf16 = 1;
  r.parts_bf16 = 1;
  (void)hipGetLastError();
  return launched(launch_reduce_ln(r, (hipStream_t)stream));
}

int tp_partial_reduce_scatter_residual_ln(const float* parts, int n_parts, int64_t part_stride,
                                          const void* residual, const void* gamma,
                                          const void* beta, float eps, void* h_out, void* y_out,
                                          int64_t rows, int64_t H, int rank, int world, int dtype,
                                          void* stream) {
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
  if (int st = check_rank(rank, world)) return st;
  if (n_parts < 0) return TP_ERR_SHAPE;
  if (n_parts > 0 && !parts) return TP_ERR_NULL;
  if (n_parts == 0 && !residual) return TP_ERR_NULL;
  if (gamma && !y_out) return TP_ERR_NULL;
  if (!gamma && !h_out) return TP_ERR_NULL;
  if (rows <= 0 || rows > INT32_MAX || H <= 0 || H > 65536) return TP_ERR_SHAPE;
  if (rows % world) return TP_ERR_DIVISIBLE;
  if (!(eps >= 0.0f) || isinf(eps)) return TP_ERR_SHAPE;
  if (n_parts > 1 && part_stride < rows * H) return TP_ERR_SHAPE;
  if (!mult8(H)) return TP_ERR_ALIGN;
  if (n_parts > 1 && (part_stride & 3)) return TP_ERR_ALIGN;
  const void* ptrs[] = {parts, residual, gamma, beta, h_out, y_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;

  // Rows [rank*rows/world, (rank+1)*rows/world) of every partial and of the residual.
  const int64_t rl = rows / world, row0 = (int64_t)rank * rl;
  const size_t es = dtype == TP_BF16 ? 2 : 4;
  ReduceDesc r;
  r.parts = parts ? parts + row0 * H : nullptr;
  r.n_parts = n_parts;
  r.part_stride = part_stride;
  r.residual = residual ? (const char*)residual + (size_t)(row0 * H) * es : nullptr;
  r.gamma = gamma;
  r.beta = beta;
  r.eps = eps;
  r.h_out = h_out;
  r.y_out = gamma ? y_out : nullptr;
  r.rows = rl;
  r.H = H;
  r.bf16 = dtype == TP_BF16;
  (void)hipGetLastError();
  return launched(launch_reduce_ln(r, (hipStream_t)stream));
}

int tp_partial_reduce_scatter_residual_ln_bf16(const void* parts, int n_parts,
                                               int64_t part_stride, const void* residual,
                                               const void* gamma, const void* beta, float eps,
                                               void* h_out, void* y_out, int64_t rows, int64_t H,
                                               int rank, int world, void* stream) {
  if (int st = check_rank(rank, world)) return st;
  if (n_parts < 0) return TP_ERR_SHAPE;
  if (n_parts > 0 && !parts) return TP_ERR_NULL;
  if (n_parts == 0 && !residual) return TP_ERR_NULL;
  if (gamma && !y_out) return TP_ERR_NULL;
  if (!gamma && !h_out) return TP_ERR_NULL;
  if (rows <= 0 || rows > INT32_MAX || H <= 0 || H > 65536) return TP_ERR_SHAPE;
  if (rows % world) return TP_ERR_DIVISIBLE;
  if (!(eps >= 0.0f) || isinf(eps)) return TP_ERR_SHAPE;
  if (n_parts > 1 && part_stride < rows * H) return TP_ERR_SHAPE;
  if (!mult8(H)) return TP_ERR_ALIGN;
  if (n_parts > 1 && !mult8(part_stride)) return TP_ERR_ALIGN;
  const void* ptrs[] = {parts, residual, gamma, beta, h_out, y_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return TP_ERR_ALIGN;

  // Rows [rank*rows/world, (rank+1)*rows/world) of every bf16 partial and of the residual.
  const int64_t rl = rows / world, row0 = (int64_t)rank * rl;
  const size_t off = (size_t)(row0 * H) * 2;
  ReduceDesc r;
  r.parts = parts ? (const float*)((const char*)parts + off) : nullptr;  // read as bf16
  r.n_parts = n_parts;
  r.part_stride = part_stride;
  r.residual = residual ? (const char*)residual + off : nullptr;
  r.gamma = gamma;
  r.beta = beta;
  r.eps = eps;
  r.h_out = h_out;
  r.y_out = gamma ? y_out : nullptr;
  r.rows = rl;
  r.H = H;
  r.bf16 = 1;
  r.parts_bf16 = 1;
  (void)hipGetLastError();
  return launched(launch_reduce_ln(r, (hipStream_t)stream));
}

}  // extern "C"
