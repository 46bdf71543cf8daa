/* tp_shard.h -- C ABI of the MI355X (gfx950) tensor-parallel layer-shard library.
 *
 * One call computes one simulated tensor-parallel rank's shard of a Megatron-style
 * Transformer layer on one GPU.  Where the layer's tensor-parallel form places an
 * all-gather between GPUs, the caller concatenates the ranks' outputs in one HBM buffer
 * (by pointing each rank's output at its column block); where it places an all-reduce,
 * the ranks' fp32 partials are stacked in HBM and summed by
 * tp_partial_reduce_residual_ln, fused with the residual add and LayerNorm, or summed in
 * place by the producing product's epilogue (the *_fold calls), or stored in bf16 and summed
 * by tp_partial_reduce_residual_ln_bf16 (the *_bf16 calls).
 *
 * Sources (web pages on tensor parallelism):
 *   typc.net "张量并行：千亿大模型突破单卡显存限制的底层技术", sections 2.1, 2.2, 3;
 *   0539edu.com TP / 3D-parallelism tutorial, sections 1.1 and 1.2 (formulas 1.1-1.13);
 *   pwwt.cn TP layout walk-through, sections 1.1-1.2 (figures 1-2), 2.1-2.3 (figures 3-5),
 *   3.1-3.4 (the weight-chunk helper and the column/row parallel layers), 5.1-5.3 and 6.3.
 *
 * Conventions shared by every call
 *   - A linear layer is Y = X.W with X [seq, H] and W [H, N] (pwwt.cn section 1.1); every
 *     matrix is row-major.  Weights are stored [in, out].
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the caller.  The
 *     library allocates nothing, frees nothing and keeps no pointer after returning.  Its one
 *     piece of device memory is the static scratch array of tp_attn_head_shard_noalloc
 *     (TP_ATTN_SCRATCH_BYTES per GPU, held from when the library's device code is loaded on
 *     that GPU until the process ends).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call is
 *     asynchronous on that stream and never synchronises.
 *   - Ranks are numbered 0..world-1; rank r owns block r of a split dimension, and rank 0
 *     owns the first block (typc.net section 2.1; pwwt.cn section 3.1).
 *   - Accumulation is always fp32.  bf16 results are rounded to nearest even.
 *   - Every argument is validated BEFORE any launch (the only HIP calls before it are
 *     queries of the current device's compute-unit count).  On error the call returns a
 *     negative tp_status, launches nothing and leaves every output untouched.  A launch
 *     failure returns TP_ERR_LAUNCH.
 *   - Alignment: pointers 16-byte aligned; leading dimensions, shard widths and the
 *     column offsets they imply are multiples of 8 elements.
 *   - Size limits: the activation operand's row width (H of the column call, ldx of the row
 *     call, H of the attention call) is at most 2^21 elements and the weight's row width (N)
 *     at most 2^23 elements; larger values return TP_ERR_SHAPE.
 *   - Calls are re-entrant; concurrent calls on different streams may not write the same
 *     output.  Results are deterministic (fixed summation order, no atomics).
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = -1,      /* a required pointer is NULL */
  TP_ERR_SHAPE = -2,     /* a size is <= 0, a leading dimension is too small, or a size is unsupported */
  TP_ERR_DIVISIBLE = -3, /* a split dimension is not a multiple of world */
  TP_ERR_RANK = -4,      /* world < 1, or rank outside [0, world) */
  TP_ERR_DTYPE = -5,     /* unknown dtype / activation, or a dtype the call does not support */
  TP_ERR_ALIGN = -6,     /* pointer, leading dimension or shard offset misaligned */
  TP_ERR_WORKSPACE = -7, /* workspace NULL or smaller than tp_attn_workspace_bytes */
  TP_ERR_LAUNCH = -8,    /* the HIP runtime reported an error at launch */
  TP_ERR_SCRATCH = -9    /* the sizes need more than the library's static scratch */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;         /* io dtype of X, W, Y, residual, LN */
typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU_TANH = 1 } tp_act;

/* Column-parallel linear with fused activation (the all-gather form).
 *
 *   Y[t, j] = act( sum_k X[t, k] * W[k, rank*N/world + j] ),  t < seq, j < N/world
 *
 * X [seq, H] dense (ld H) is the full input every rank holds; W [H, N] dense (ld N) is the
 * full weight, of which rank `rank` uses the column block [rank*N/world, (rank+1)*N/world)
 * (typc.net section 2.1; 0539edu.com section 1.1 "column split", figure 1.2; pwwt.cn
 * sections 1.1 and 3.2).  Y receives the N/world output columns with leading dimension
 * ldy >= N/world.  To concatenate the simulated ranks' outputs (the all-gather) pass
 * Y = Yfull + rank*N/world and ldy = N.  act is tp_act: GeLU with the tanh form
 *   0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 * is applied per element before rounding to the io dtype (0539edu.com section 1.2.1: the
 * elementwise activation commutes with the column split).  dtype TP_BF16 or TP_F32.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE (seq, H, N <= 0 or ldy < N/world), TP_ERR_DIVISIBLE
 * (N % world), TP_ERR_RANK, TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_LAUNCH. */
int tp_col_linear_gelu(const void* X, const void* W, void* Y, int64_t ldy,
                       int64_t seq, int64_t H, int64_t N, int rank, int world,
                       int act, int dtype, void* stream);

/* Row-parallel linear, partial sum of one rank (the all-reduce form, before the reduce).
 *
 *   Zpart[t, n] = sum_{k < K/world} X[t, k] * W[rank*K/world + k, n]
 *
 * X is the rank's input shard x_partial [seq, K/world] with leading dimension
 * ldx >= K/world: the row-parallel layer takes the partial input, not the full one
 * (pwwt.cn section 3.3, RowParallelLinear.forward(x_partial)).  For the MLP this is exactly
 * the block the rank's column-parallel call wrote, which stays on the rank (the column ->
 * row pairing needs no exchange in between; 0539edu.com section 1.2.1).  If the input is
 * held as one concatenated [seq, K] buffer, pass X = Xfull + rank*K/world and ldx = K.
 * W [K, N] dense (ld N) is the full weight; rank `rank` uses its row block
 * [rank*K/world, (rank+1)*K/world) (typc.net section 2.2; 0539edu.com section 1.1
 * formula 1.1 "outer-product-sum split"; pwwt.cn sections 1.2 and 3.3).  Zpart [seq, N] is
 * dense fp32 whatever the io dtype; the full result is the sum of all ranks' partials.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE (ldx < K/world), TP_ERR_DIVISIBLE (K % world),
 * TP_ERR_RANK, TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_LAUNCH. */
int tp_row_linear_partial(const void* X, int64_t ldx, const void* W, float* Zpart,
                          int64_t seq, int64_t K, int64_t N, int rank, int world,
                          int dtype, void* stream);

/* Row-parallel linear with the reduce folded into the product's epilogue (pwwt.cn section
 * 2.3: fusing the all-reduce with the residual add; section 5.3: fusion as the first way to
 * save exchange).  The ranks' partials are summed in place as they are produced instead of
 * being stacked and reduced afterwards:
 *
 *   accumulate == 0:  Zsum[t, n]  = sum_{k < K/world} X[t, k] * W[rank*K/world + k, n]
 *   accumulate != 0:  Zsum[t, n] += sum_{k < K/world} X[t, k] * W[rank*K/world + k, n]
 *
 * Arguments, shard addressing and errors are those of tp_row_linear_partial, with Zsum
 * [seq, N] dense fp32 in place of Zpart; Zsum must not overlap X or W.  Calling rank 0 with
 * accumulate == 0 and then ranks 1..world-1 with accumulate != 0, in that order on one stream,
 * leaves Zsum = ((Z_0 + Z_1) + ...) + Z_{world-1} in fp32, the same additions in the same
 * order as tp_partial_reduce_residual_ln applies to the stacked partials.  Passing Zsum to
 * that call with n_parts = 1 therefore gives bit-identical h and y, while the reduce reads
 * one fp32 [seq, N] block instead of world of them and the stacked buffer is not needed. */
int tp_row_linear_fold(const void* X, int64_t ldx, const void* W, float* Zsum,
                       int64_t seq, int64_t K, int64_t N, int rank, int world,
                       int accumulate, int dtype, void* stream);

/* Row-parallel linear with bf16 partials, the exchange as the pages count it (pwwt.cn
 * section 5.2: the all-reduce's [S, H] input at 2 bytes per element, BF16; section 6.3: the
 * summation order and BF16 arithmetic as sources of error between TP and one device).
 * Zpart[t, n] is the fp32 sum of tp_row_linear_partial,
 * rounded once to bf16 (nearest, ties to even) and written as a dense bf16 [seq, N] block;
 * tp_partial_reduce_residual_ln_bf16 then reads half the bytes of the fp32 partials.  The
 * partials' rounding adds to the error of the reduced sum (relative to its partials, 2^-8 per
 * partial), so this is a variant beside the fp32-partial path, not a replacement.  Inputs are
 * bf16 (no dtype argument); X, ldx, W, shard addressing and errors are those of
 * tp_row_linear_partial (TP_ERR_DTYPE does not occur). */
int tp_row_linear_partial_bf16(const void* X, int64_t ldx, const void* W, void* Zpart,
                               int64_t seq, int64_t K, int64_t N, int rank, int world,
                               void* stream);

/* Column-parallel linear + GeLU that also keeps the pre-activation for the backward pass:
 * exactly tp_col_linear_gelu with act = TP_ACT_GELU_TANH, plus
 *
 *   U[t, j] = sum_k X[t, k] * W[k, rank*N/world + j]     rounded to bf16, ld ldu >= N/world
 *
 * (U is what the GeLU's derivative is evaluated at in tp_row_linear_backward; Y is computed
 * from the fp32 sum, not from the rounded U).  Only dtype TP_BF16.
 * Errors: as tp_col_linear_gelu, TP_ERR_NULL for U, TP_ERR_SHAPE for ldu < N/world. */
int tp_col_linear_gelu_save(const void* X, const void* W, void* Y, int64_t ldy, void* U,
                            int64_t ldu, int64_t seq, int64_t H, int64_t N, int rank, int world,
                            int dtype, void* stream);

/* Backward of the row-parallel linear of rank `rank`, with the derivative of the activation
 * that precedes it (the column layer's GeLU) fused in.  The pages state that the backward
 * pass has its own communication pattern and that the gradients are sharded like the
 * weights (typc.net section 2.2; pwwt.cn sections 1.3 and 6.1), without formulas; these are
 * the chain rule applied to Zpart = Y_r . W_r, Z = sum_r Zpart_r:
 *
 *   dY[t, j]  = act'(U[t, j]) * sum_n dZ[t, n] * W[rank*K/world + j, n]     (dZ . W_r^T)
 *   dW[j, n] (+)= sum_t Y[t, j] * dZ[t, n]                                 (Y_r^T . dZ)
 *
 * for t < seq, j < K/world, n < N.  The forward all-reduce turns into an identity: every rank
 * uses the full dZ [seq, N] (dense, ld N), so this call needs no exchange.  W [K, N] dense is
 * the full weight (row block `rank` is used).  Y [seq, K/world] (ld ldy) is the rank's
 * forward input shard; U [seq, K/world] (ld ldu) the pre-activation of the column layer that
 * produced Y (tp_col_linear_gelu_save), used only with act = TP_ACT_GELU_TANH (act'(u) is
 * the tanh-form GeLU's derivative; with TP_ACT_NONE act' = 1 and U may be NULL).  Outputs:
 * dY bf16 [seq, K/world] (ld ld_dy >= K/world), the gradient at the rank's column-layer
 * output; dW fp32 [K/world, N] (ld ld_dw >= N), the gradient of the rank's row block of W,
 * overwritten, or added to when accumulate != 0 (gradient accumulation over micro-batches).
 * Either output may be NULL to skip its product (not both).  Only dtype TP_BF16.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE (sizes <= 0, seq > 2^30, a leading dimension too small,
 * N or ldy > 2^21), TP_ERR_DIVISIBLE (K % world), TP_ERR_RANK, TP_ERR_DTYPE, TP_ERR_ALIGN,
 * TP_ERR_LAUNCH. */
int tp_row_linear_backward(const void* dZ, const void* W, const void* Y, int64_t ldy,
                           const void* U, int64_t ldu, void* dY, int64_t ld_dy, float* dW,
                           int64_t ld_dw, int64_t seq, int64_t K, int64_t N, int rank, int world,
                           int act, int accumulate, int dtype, void* stream);

/* Backward of the column-parallel linear of rank `rank` (chain rule on Y_r = X . W_r, the
 * rank's column block):
 *
 *   dXpart[t, h] = sum_j dU[t, j] * W[h, rank*N/world + j]                 (dU_r . W_r^T)
 *   dW[h, j]   (+)= sum_t X[t, h] * dU[t, j]                              (X^T . dU_r)
 *
 * for t < seq, h < H, j < N/world.  X [seq, H] dense is the full forward input, W [H, N]
 * dense the full weight (column block `rank` is used), dU [seq, N/world] (ld ldu) the
 * gradient at the rank's pre-activation output (dY of tp_row_linear_backward).  dXpart fp32
 * [seq, H] dense is this rank's partial of the input gradient: the forward identity turns
 * into an all-reduce, dX = sum over ranks of dXpart, which tp_partial_reduce_residual_ln
 * computes from the stacked partials (gamma = NULL, residual = the gradient arriving along
 * the residual path or NULL).  dW fp32 [H, N/world] (ld ld_dw >= N/world) is the gradient
 * of the rank's column block, overwritten or (accumulate != 0) added to.  Either output may
 * be NULL (not both).  Only dtype TP_BF16.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE (sizes <= 0, seq > 2^30, a leading dimension too small,
 * H, N or ldu > 2^21), TP_ERR_DIVISIBLE (N % world), TP_ERR_RANK, TP_ERR_DTYPE, TP_ERR_ALIGN,
 * TP_ERR_LAUNCH. */
int tp_col_linear_backward(const void* X, const void* W, const void* dU, int64_t ldu,
                           float* dXpart, float* dW, int64_t ld_dw, int64_t seq, int64_t H,
                           int64_t N, int rank, int world, int accumulate, int dtype,
                           void* stream);

/* tp_col_linear_backward with the input-gradient partial exchanged in bf16, as the forward
 * partials of tp_row_linear_partial_bf16 are (pwwt.cn section 5.2 counts the all-reduce's
 * [S, H] operand at 2 bytes per element; section 6.3 names BF16 and the summation order as
 * the sources of error between TP and one device).  dXpart bf16 [seq, H] dense receives the
 * fp32 sum of tp_col_linear_backward's dXpart, rounded once to bf16 (nearest, ties to even);
 * tp_partial_reduce_residual_ln_bf16 (gamma = NULL) then sums the ranks' partials.  dW, the
 * other arguments and the errors are those of tp_col_linear_backward with dtype TP_BF16 (no
 * dtype argument, so no TP_ERR_DTYPE). */
int tp_col_linear_backward_bf16(const void* X, const void* W, const void* dU, int64_t ldu,
                                void* dXpart, float* dW, int64_t ld_dw, int64_t seq, int64_t H,
                                int64_t N, int rank, int world, int accumulate, void* stream);

/* Workspace bytes tp_attn_head_shard needs for these sizes on the current device; 0 if the
 * sizes are invalid.  It queries the device's compute-unit count (the QKV projection's launch
 * plan, and with it the size of the split-strip partials below, depends on it), so call it
 * with the device current that the attention call will run on. */
size_t tp_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t H, int n_heads,
                               int head_dim, int world, int dtype);

/* Attention-head shard of one rank: column-split QKV projection, per-head softmax
 * attention over the rank's heads, row-split output projection (0539edu.com section 1.2.2,
 * formulas 1.8-1.13, figure 1.5; pwwt.cn section 2.2, figure 4; typc.net section 3).
 *
 *   heads of rank r: [r*n_heads/world, (r+1)*n_heads/world), hl = n_heads/world, d = head_dim
 *   Q_r | K_r | V_r  = Xn . Wqkv[:, column blocks of those heads]          [T, 3*hl*d]
 *   O_h = softmax(Q_h K_h^T / sqrt(d) + causal mask) V_h   per sequence and head
 *   A_r = concat of O_h over the rank's heads, ascending                  [T, hl*d]
 *   Zpart = A_r . Wo[r*hl*d : (r+1)*hl*d, :]                              [T, H] fp32
 *
 * Xn [batch*seq, H] dense: the (already normalised) input, sequences contiguous.  Wqkv
 * [H, 3H] dense = [Wq | Wk | Wv], head h owning columns [h*d, (h+1)*d) of each block.  Wo
 * [H, H] dense.  H must equal n_heads*head_dim; head_dim must be 128; seq < 2^30 and
 * batch*seq < 2^31 (TP_ERR_SHAPE otherwise).  causal: key j is
 * visible to query i iff j <= i within the same sequence.  Only dtype TP_BF16.
 * workspace (device, >= tp_attn_workspace_bytes, 256-byte aligned) receives, as a
 * documented by-product, QKV_r bf16 [T, 3*hl*d] at offset 0 and A_r bf16 [T, hl*d] right
 * after it (offset T*3*hl*d*2 bytes).  When the QKV projection's launch plan has a narrow
 * strip of columns (those that do not fill a whole round of 256 x 256 tiles on this device),
 * the strip's contraction is split over 4 ranges whose fp32 partials follow A_r in the
 * workspace and are summed in range order into QKV_r; the rest of QKV_r is one fp32
 * accumulation per element.  Results are deterministic for a given device.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_DIVISIBLE (n_heads % world), TP_ERR_RANK,
 * TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_WORKSPACE, TP_ERR_LAUNCH. */
int tp_attn_head_shard(const void* Xn, const void* Wqkv, const void* Wo, float* Zpart,
                       int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                       int rank, int world, int causal, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Attention-head shard with the reduce folded into the output projection's epilogue, as
 * tp_row_linear_fold does for the row-parallel linear: the rank's A_r . Wo[rank rows, :] is
 * written to Zsum [batch*seq, H] fp32 when accumulate == 0 and added to it otherwise.  All
 * other arguments, the workspace contents and the errors are those of tp_attn_head_shard;
 * Zsum must not overlap Xn, Wqkv, Wo or the workspace. */
int tp_attn_head_shard_fold(const void* Xn, const void* Wqkv, const void* Wo, float* Zsum,
                            int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                            int rank, int world, int causal, int accumulate, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Attention-head shard with a bf16 partial (the bf16-partial variant of
 * tp_row_linear_partial_bf16 for the output projection): Zpart [batch*seq, H] receives the
 * fp32 A_r . Wo[rank rows, :] of tp_attn_head_shard rounded once to bf16.  Inputs are bf16
 * (no dtype argument); all other arguments, the workspace contents and the errors are those
 * of tp_attn_head_shard. */
int tp_attn_head_shard_bf16(const void* Xn, const void* Wqkv, const void* Wo, void* Zpart,
                            int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                            int rank, int world, int causal, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of the library's own scratch array (one per GPU) that tp_attn_head_shard_noalloc uses
 * as its workspace: 160 MiB, what tp_attn_workspace_bytes gives for one rank of the largest
 * workload served (8192 tokens, 12 heads of 128 per rank, H = 12288, on 256 compute units:
 * QKV_r 75.5 MB + A_r 25.2 MB + the split strip's fp32 partials 67.1 MB). */
#define TP_ATTN_SCRATCH_BYTES ((size_t)160 << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): tp_attn_head_shard without the workspace argument.
 * The workspace is taken from a static device array of TP_ATTN_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call itself allocates nothing
 * (no hipMalloc or hipFree, no allocating library routine).  Its first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress), which loads the library's device
 * code there if it is not loaded yet: make one call on each device before capturing a graph.
 * Arguments, results and errors are those of tp_attn_head_shard, with the outputs
 * bit-identical to it for the same inputs, except:
 *   - sizes whose tp_attn_workspace_bytes exceeds TP_ATTN_SCRATCH_BYTES return TP_ERR_SCRATCH
 *     (before any launch);
 *   - every call on one GPU shares that GPU's array, which keeps the last call's QKV_r and
 *     A_r: calls that overlap in time on one GPU (on different streams, or from different
 *     threads without ordering) race and give undefined results.  Order them on one stream.
 *     No part of the array needs clearing: every byte a call reads it wrote first.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_DIVISIBLE, TP_ERR_RANK, TP_ERR_DTYPE,
 * TP_ERR_ALIGN, TP_ERR_SCRATCH, TP_ERR_LAUNCH (also when the array's address cannot be
 * obtained on the current device). */
int tp_attn_head_shard_noalloc(const void* Xn, const void* Wqkv, const void* Wo, float* Zpart,
                               int64_t batch, int64_t seq, int64_t H, int n_heads, int head_dim,
                               int rank, int world, int causal, int dtype, void* stream);

/* The all-reduce replacement, fused with the residual add and LayerNorm (pwwt.cn section
 * 2.3: the single all-reduce sits just before the residual add, and fusing it with the
 * residual add or the next LayerNorm's statistics; section 6.3: residual + LayerNorm as
 * one fused op with a consistent statistics order).  Over `rows` rows of width H:
 *
 *   h = residual + sum_{p = 0}^{n_parts-1} parts[p * part_stride + ...]   fp32, p ascending
 *   y = (h - mean(h)) / sqrt(var(h) + eps) * gamma + beta    biased var, fp32 statistics of h
 *
 * parts: n_parts dense fp32 [rows, H] blocks, block p starting at parts + p*part_stride
 * (part_stride >= rows*H elements).  n_parts == 0 gives a plain LayerNorm of `residual`
 * (parts may then be NULL).  residual may be NULL (treated as 0); h_out may be NULL;
 * gamma == NULL skips the LayerNorm (y_out is then ignored); beta == NULL means 0.
 * residual, gamma, beta, h_out and y_out use `dtype`; h_out and y_out must not alias the
 * parts.  Requires H % 8 == 0, H <= 65536 and 1 <= rows < 2^31.
 * Errors: TP_ERR_NULL (no input at all, or gamma given with y_out NULL), TP_ERR_SHAPE,
 * TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_LAUNCH. */
int tp_partial_reduce_residual_ln(const float* parts, int n_parts, int64_t part_stride,
                                  const void* residual, const void* gamma, const void* beta,
                                  float eps, void* h_out, void* y_out,
                                  int64_t rows, int64_t H, int dtype, void* stream);

/* tp_partial_reduce_residual_ln over bf16 partials (those of tp_row_linear_partial_bf16 and
 * tp_attn_head_shard_bf16): each partial is widened to fp32 and the sum, residual add and
 * LayerNorm are those of the fp32-partial call, in the same order.  parts: n_parts dense bf16
 * [rows, H] blocks, block p at parts + p*part_stride elements (part_stride >= rows*H and a
 * multiple of 8 when n_parts > 1).  residual, gamma, beta, h_out and y_out are bf16.  Other
 * arguments and errors are those of tp_partial_reduce_residual_ln (no dtype argument, so no
 * TP_ERR_DTYPE). */
int tp_partial_reduce_residual_ln_bf16(const void* parts, int n_parts, int64_t part_stride,
                                       const void* residual, const void* gamma, const void* beta,
                                       float eps, void* h_out, void* y_out,
                                       int64_t rows, int64_t H, void* stream);

/* Sequence-parallel form of the same epilogue: the reduce-scatter of rank `rank`, fused with
 * the residual add and LayerNorm of that rank's rows (pwwt.cn section 5.1, figure 7: an
 * all-reduce is a reduce-scatter followed by an all-gather, and a consumer that needs only
 * its share of the rows can take the reduce-scatter result directly; section 5.3: Megatron's
 * sequence parallelism splits along the sequence, so each rank holds [S/P, H] instead of
 * [S, H]).  With rl = rows/world and row0 = rank*rl:
 *
 *   h[i] = residual[row0 + i] + sum_{p ascending} parts[p][row0 + i]     i < rl, fp32
 *   y[i] = LayerNorm(h[i]) * gamma + beta
 *
 * parts, n_parts, part_stride and residual describe the FULL [rows, H] operands, exactly as
 * for tp_partial_reduce_residual_ln; h_out and y_out receive the rank's rl rows (dense,
 * [rl, H]).  Pointing them at row row0 of full [rows, H] buffers for every rank is the
 * all-gather (concatenation along rows).  Each output row is computed by the same arithmetic
 * as the corresponding row of tp_partial_reduce_residual_ln, so the results are identical.
 * Errors: as tp_partial_reduce_residual_ln, plus TP_ERR_RANK and TP_ERR_DIVISIBLE
 * (rows % world). */
int tp_partial_reduce_scatter_residual_ln(const float* parts, int n_parts, int64_t part_stride,
                                          const void* residual, const void* gamma,
                                          const void* beta, float eps, void* h_out, void* y_out,
                                          int64_t rows, int64_t H, int rank, int world, int dtype,
                                          void* stream);

/* The sequence-parallel epilogue over bf16 partials: tp_partial_reduce_scatter_residual_ln's
 * rows of rank `rank`, with the partials, the residual and the outputs in bf16 as for
 * tp_partial_reduce_residual_ln_bf16 (part_stride a multiple of 8 when n_parts > 1).  Each
 * output row is computed by the same arithmetic as the corresponding row of
 * tp_partial_reduce_residual_ln_bf16.  Errors: as tp_partial_reduce_residual_ln_bf16, plus
 * TP_ERR_RANK and TP_ERR_DIVISIBLE (rows % world). */
int tp_partial_reduce_scatter_residual_ln_bf16(const void* parts, int n_parts,
                                               int64_t part_stride, const void* residual,
                                               const void* gamma, const void* beta, float eps,
                                               void* h_out, void* y_out, int64_t rows, int64_t H,
                                               int rank, int world, void* stream);

/* Static, NUL-terminated description of a tp_status value. */
const char* tp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
