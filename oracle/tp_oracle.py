"""Plain float64 CPU oracle of one rank's shard of a tensor-parallel Transformer layer.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Never used by the product path.

Sources (the four web pages on tensor parallelism; cited by site and section):
  [typc]  typc.net, "张量并行：千亿大模型突破单卡显存限制的底层技术"
  [edu]   0539edu.com, tensor parallelism and 3D parallelism tutorial
  [pwwt]  pwwt.cn, tensor-parallel layout walk-through with hand-written TP layers
  [qwen]  qianwenai.com, "什么是张量并行"

Conventions.  A linear layer is Y = X.W with X [seq, H], W [H, N] ([pwwt] section
1.1, figure 1), weights stored [in, out] row-major.  Ranks are numbered from 0 and
rank 0 owns the first block ([typc] section 2.1).  Inputs are the exact float32
values of the generated tensors (bf16 inputs decoded exactly); every product and
sum is evaluated in float64 and no intermediate is rounded back to bf16.  The
matrix product is numpy's float64 ``@`` (a library primitive); everything else is
written out.

Readings of passages the pages leave open (listed with reasons in the design notes):
  * weights [in, out]; column split = dim 1, row split = dim 0;
  * a dimension that the world size does not divide is rejected, not floored;
  * activation = GeLU with the tanh approximation;
  * fused QKV weight = [Wq | Wk | Wv], head h owning columns [h*d, (h+1)*d) of each;
  * attention scale 1/sqrt(head_dim), causal = key j visible to query i iff j <= i
    within one sequence;
  * partials summed in ascending rank order, then the residual added;
  * LayerNorm: biased variance, eps = 1e-5, affine after normalising; no bias, no
    dropout anywhere.

Every function below is pinned by tests in tests/test_oracle_pins.py (closed forms,
integer-exact identities, brute force on tiny inputs, and library routines for the
special cases that reduce to them); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "shard_range", "matmul", "gelu_tanh", "col_linear", "concat_columns",
    "row_linear_partial", "reduce_partials", "layer_norm", "reduce_residual_layernorm",
    "split_qkv", "head_range", "attention_heads", "attn_head_shard", "mlp_shard",
    "block_shard", "block_forward", "reduce_scatter_rows", "reduce_scatter_residual_layernorm",
    "concat_rows", "gelu_tanh_grad", "row_linear_backward", "col_linear_backward",
    "mlp_shard_backward", "mlp_backward", "round_bf16", "row_linear_partial_bf16",
    "attn_head_shard_bf16", "col_linear_backward_bf16",
]

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------- sharding
def shard_range(n: int, world: int, rank: int) -> Tuple[int, int]:
    """Block ``rank`` of ``world`` equal contiguous blocks of a length-n dimension.

    [pwwt] section 3.1 (the weight-chunk helper: block size = size // world, block of
    rank r starts at r * size); [typc] section 2.1 (W 4096x8192 split into two halves
    of columns, GPU0 holding the first 4096).  A remainder is rejected instead of
    silently dropped.
    """
    if world < 1:
        raise ValueError("world must be >= 1")
    if not 0 <= rank < world:
        raise ValueError("rank out of range")
    if n % world:
        raise ValueError(f"dimension {n} not divisible by world {world}")
    c = n // world
    return rank * c, (rank + 1) * c


def matmul(a, b) -> np.ndarray:
    """Float64 matrix product (library primitive)."""
    return _f64(a) @ _f64(b)


# ----------------------------------------------------------------------------- activation
def gelu_tanh(x) -> np.ndarray:
    """GeLU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).

    The pages name "ReLU or GeLU" as the elementwise activation between the two MLP
    linears ([edu] section 1.2.1); the tanh form is the one the workloads fix.
    """
    x = _f64(x)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x * x * x)))


def _act(y: np.ndarray, act: str) -> np.ndarray:
    if act == "none":
        return y
    if act == "gelu_tanh":
        return gelu_tanh(y)
    raise ValueError(act)


def gelu_tanh_grad(x) -> np.ndarray:
    """Derivative of gelu_tanh, by the chain rule.  With c = sqrt(2/pi), a = 0.044715 and
    u = c (x + a x^3):

      d/dx [0.5 x (1 + tanh u)] = 0.5 (1 + tanh u) + 0.5 x (1 - tanh(u)^2) c (1 + 3 a x^2).

    Needed by the backward pass of the MLP pair, which the pages mention without formulas
    ([typc] section 2.2; [pwwt] sections 1.3 and 6.1).
    """
    x = _f64(x)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (x + 0.044715 * x * x * x))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x)


def _act_grad(u: np.ndarray, act: str) -> np.ndarray:
    if act == "none":
        return np.ones_like(_f64(u))
    if act == "gelu_tanh":
        return gelu_tanh_grad(u)
    raise ValueError(act)


# ----------------------------------------------------------------------------- linears
def col_linear(X, W, rank: int, world: int, act: str = "none",
               rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Column-parallel linear, rank r's output block: act(X . W[:, block r]).

    X is the full (replicated) input [seq, H]; W [H, N] is split along its output
    dimension N ([typc] section 2.1; [edu] section 1.1 figure 1.2 "column split";
    [pwwt] section 1.1 figure 1 and section 3.2).  The elementwise activation is
    applied per shard, since it commutes with the column split ([edu] section 1.2.1).
    ``rows`` restricts the computation to those rows of X (rows are independent).
    """
    n0, n1 = shard_range(W.shape[1], world, rank)
    if X.shape[1] != W.shape[0]:
        raise ValueError("inner dimensions differ")
    Xs = X if rows is None else X[np.asarray(rows)]
    return _act(matmul(Xs, W[:, n0:n1]), act)


def concat_columns(blocks: Sequence[np.ndarray]) -> np.ndarray:
    """The all-gather of column shards: blocks concatenated along the last dimension
    in ascending rank order ([pwwt] section 3.2: gathered outputs are ordered by rank
    and concatenated on the last dim; [edu] section 1.1 figure 1.2)."""
    return np.concatenate([_f64(b) for b in blocks], axis=-1)


def row_linear_partial(X, W, rank: int, world: int,
                       rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Row-parallel linear, rank r's partial sum: X[:, block r] . W[block r, :].

    X is the full input [seq, K] whose column block r is the rank's input shard; W
    [K, N] is split along its input dimension K ([typc] section 2.2; [edu] section
    1.1 formula 1.1 "outer-product-sum split"; [pwwt] section 1.2 figure 2 and
    section 3.3).  The full output is the sum of all ranks' partials.
    """
    if X.shape[1] != W.shape[0]:
        raise ValueError("inner dimensions differ")
    k0, k1 = shard_range(W.shape[0], world, rank)
    Xs = X if rows is None else X[np.asarray(rows)]
    return matmul(Xs[:, k0:k1], W[k0:k1, :])


def reduce_partials(parts: Sequence[np.ndarray]) -> np.ndarray:
    """The all-reduce of row-parallel partials: elementwise sum in ascending rank
    order ([typc] section 2.2; [pwwt] section 1.2; a fixed summation order per
    [pwwt] section 6.3)."""
    if len(parts) == 0:
        raise ValueError("no partials")
    acc = np.array(_f64(parts[0]), copy=True)
    for p in parts[1:]:
        acc += _f64(p)
    return acc


def round_bf16(x) -> np.ndarray:
    """x rounded to the nearest bfloat16 value, ties to even, returned in float64.

    bfloat16 keeps float32's exponent range and 8 significant bits: a normal value
    2^e * 1.f has the quantum 2^(e-7); below the smallest normal 2^-126 the quantum stays
    2^-133 (subnormals).  The quotient x / quantum is an exact float64 (a power-of-two
    scaling), so one round-half-to-even of it is the correctly rounded result.  Values whose
    rounded magnitude exceeds the largest bfloat16 (2 - 2^-7) * 2^127 become infinities."""
    x = _f64(x)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                      # x = m * 2^e with 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)  # the quantum at x's binade
    r = np.rint(x[fin] / q) * q
    big = np.abs(r) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    out[~fin] = x[~fin]                          # zeros (with their sign), infinities, NaN
    return out


def row_linear_partial_bf16(X, W, rank: int, world: int,
                            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rank r's row-parallel partial as it is exchanged in bf16: row_linear_partial rounded
    once to bfloat16.  [pwwt] section 5.2 counts the all-reduce's [S, H] input at 2 bytes per
    element (BF16), and section 6.3 names BF16 arithmetic and the summation order as where
    tensor-parallel results part from one device's."""
    return round_bf16(row_linear_partial(X, W, rank, world, rows))


def row_linear_fold(Zsum, X, W, rank: int, world: int, accumulate: bool) -> np.ndarray:
    """The reduce folded into the row-parallel product: rank r's partial is added to the
    running sum Zsum as it is produced (accumulate), or starts it (rank 0, not accumulate),
    instead of being kept for a separate reduce.  This is the fusion of the all-reduce with
    its producer that [pwwt] section 2.3 (figure 5, fusing the all-reduce with the residual
    add) and section 5.3 (fusion as the first saving) describe.  Folding ranks 0..P-1 in
    ascending order performs the same additions as reduce_partials."""
    part = row_linear_partial(X, W, rank, world)
    if not accumulate:
        return part
    return _f64(Zsum) + part


# ----------------------------------------------------------------------------- backward
# The pages say that the backward pass of the split linears has its own communication
# pattern and that each rank computes only the gradient of its own block of W, a gradient as
# sharded as the weight ([typc] section 2.2; [pwwt] section 1.3; the troubleshooting table of
# [pwwt] section 6.1 names the transposed-weight dimensions and the rank order of the
# gradient split), but give no formulas.  The functions below are the chain rule applied to
# the forward definitions above, for a loss L whose gradient at the layer output is dZ:
#   Z = Y . W      =>  dL/dY = dZ . W^T,  dL/dW = Y^T . dZ.
def row_linear_backward(dZ, Y, W, rank: int, world: int, U=None,
                        act: str = "none") -> Tuple[np.ndarray, np.ndarray]:
    """Backward of the row-parallel linear of rank r (Zpart_r = Y_r . W[block r, :],
    Z = sum_r Zpart_r).  Every rank receives the full dZ [seq, N] (the forward all-reduce
    is an identity in the backward pass).  Returns (dY_r, dW_r):

      dY_r = (dZ . W[block r, :]^T) * act'(U_r)     [seq, K/world]
      dW_r = Y_r^T . dZ                             [K/world, N]

    Y_r [seq, K/world] is the rank's forward input; when Y_r = act(U_r) came from the
    column layer, the factor act'(U_r) turns dY_r into the gradient at the pre-activation
    U_r (act "none": factor 1, U unused).
    """
    k0, k1 = shard_range(W.shape[0], world, rank)
    W = _f64(W)
    dZ = _f64(dZ)
    Y = _f64(Y)
    if Y.shape != (dZ.shape[0], k1 - k0) or dZ.shape[1] != W.shape[1]:
        raise ValueError("shapes differ")
    dY = matmul(dZ, W[k0:k1, :].T)
    if act != "none":
        dY = dY * _act_grad(U, act)
    return dY, matmul(Y.T, dZ)


def col_linear_backward(dU, X, W, rank: int, world: int) -> Tuple[np.ndarray, np.ndarray]:
    """Backward of the column-parallel linear of rank r (U_r = X . W[:, block r]).  Returns
    (dX_part_r, dW_r):

      dX_part_r = dU_r . W[:, block r]^T      [seq, H]
      dW_r      = X^T . dU_r                   [H, N/world]

    The full dX is the sum of dX_part_r over the ranks: the forward identity (every rank
    reads the whole X) becomes an all-reduce in the backward pass.
    """
    n0, n1 = shard_range(W.shape[1], world, rank)
    X = _f64(X)
    dU = _f64(dU)
    if dU.shape != (X.shape[0], n1 - n0) or X.shape[1] != W.shape[0]:
        raise ValueError("shapes differ")
    return matmul(dU, _f64(W)[:, n0:n1].T), matmul(X.T, dU)


def col_linear_backward_bf16(dU, X, W, rank: int, world: int) -> Tuple[np.ndarray, np.ndarray]:
    """col_linear_backward with the input-gradient partial exchanged in bf16: dX_part_r
    rounded once to bfloat16, dW_r unchanged.  The backward all-reduce carries an [S, H]
    operand like the forward one, which [pwwt] section 5.2 counts at 2 bytes per element."""
    dX_part, dW = col_linear_backward(dU, X, W, rank, world)
    return round_bf16(dX_part), dW


def mlp_shard_backward(X, A, B, dZ, rank: int, world: int, act: str = "gelu_tanh",
                       bf16_dx_partials: bool = False) -> Dict:
    """Rank r's backward of mlp_shard: forward U_r = X . A[:, block r], Y_r = act(U_r), then
    the row layer's backward (fused with act') and the column layer's backward
    (col_linear_backward_bf16 when bf16_dx_partials).  Returns {"U", "Y", "dU", "dB", "dA",
    "dX_part"}: dB is the gradient of B[block r, :], dA of A[:, block r], dX_part the rank's
    partial of the input gradient."""
    U = col_linear(X, A, rank, world, "none")
    Y = _act(U, act)
    dU, dB = row_linear_backward(dZ, Y, B, rank, world, U, act)
    col_bwd = col_linear_backward_bf16 if bf16_dx_partials else col_linear_backward
    dX_part, dA = col_bwd(dU, X, A, rank, world)
    return {"U": U, "Y": Y, "dU": dU, "dB": dB, "dA": dA, "dX_part": dX_part}


def mlp_backward(X, A, B, dZ, world: int, act: str = "gelu_tanh",
                 bf16_dx_partials: bool = False) -> Dict:
    """Backward of the whole tensor-parallel MLP: every rank's mlp_shard_backward, then
    dX = sum of the partials (ascending ranks), dA = the column blocks concatenated, dB = the
    row blocks stacked, in rank order.  Returns {"dX", "dA", "dB"}."""
    shards = [mlp_shard_backward(X, A, B, dZ, r, world, act, bf16_dx_partials)
              for r in range(world)]
    return {"dX": reduce_partials([s["dX_part"] for s in shards]),
            "dA": concat_columns([s["dA"] for s in shards]),
            "dB": concat_rows([s["dB"] for s in shards])}


# ----------------------------------------------------------------------------- LayerNorm
def layer_norm(h, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last dimension: (h - mean) / sqrt(var + eps) * gamma + beta,
    with the biased (population) variance computed in two passes.

    The pages place LayerNorm before attention and before the MLP ([pwwt] section 2.1
    figure 3) and fuse it with the residual add ([pwwt] sections 2.3, 5.3, 6.3); its
    formula and eps are not given, so the textbook definition is used.
    """
    h = _f64(h)
    mu = h.mean(axis=-1, keepdims=True)
    c = h - mu
    var = (c * c).mean(axis=-1, keepdims=True)
    y = c / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    if beta is not None:
        y = y + _f64(beta)
    return y


def reduce_residual_layernorm(parts: Sequence[np.ndarray], residual=None, gamma=None,
                              beta=None, eps: float = 1e-5):
    """The all-reduce replacement fused with residual add and LayerNorm:
    h = residual + sum_r parts[r] (ascending r); y = LayerNorm(h) when gamma is given.

    [pwwt] section 2.3 (the MLP's single all-reduce sits right before the residual
    add; fusing the all-reduce with the residual add or the next LayerNorm's
    statistics) and section 6.3 (residual + LayerNorm fused with a consistent
    statistics order).  With no partials this is a plain LayerNorm of ``residual``.
    Returns (h, y); y is None when gamma is None.
    """
    if len(parts) == 0 and residual is None:
        raise ValueError("nothing to reduce")
    h = reduce_partials(parts) if len(parts) else np.zeros_like(_f64(residual))
    if residual is not None:
        h = h + _f64(residual)
    y = layer_norm(h, gamma, beta, eps) if gamma is not None else None
    return h, y


def reduce_scatter_rows(parts: Sequence[np.ndarray], rank: int, world: int) -> np.ndarray:
    """The reduce-scatter half of the all-reduce, split along the rows (the sequence): rank
    r receives the sum over ranks (ascending) of row block r of every partial.

    [pwwt] section 5.1, figure 7: an all-reduce is a reduce-scatter, after which each rank
    holds one block of the summed tensor, followed by an all-gather of those blocks; a
    consumer that needs only its block can take the reduce-scatter result directly.
    Section 5.3: Megatron's sequence parallelism makes that block a block of the sequence,
    [S/P, H] per rank.
    """
    if len(parts) == 0:
        raise ValueError("no partials")
    lo, hi = shard_range(_f64(parts[0]).shape[0], world, rank)
    return reduce_partials([_f64(p)[lo:hi] for p in parts])


def reduce_scatter_residual_layernorm(parts: Sequence[np.ndarray], residual, gamma, beta,
                                      eps: float, rank: int, world: int):
    """Sequence-parallel epilogue of rank r: its row block of the summed partials, plus the
    same rows of the residual, then LayerNorm of those rows (the residual add and
    LayerNorm act on each rank's share of the sequence; [pwwt] sections 5.1 and 5.3).
    Returns (h_r, y_r); y_r is None when gamma is None."""
    h = reduce_scatter_rows(parts, rank, world) if len(parts) else None
    if residual is not None:
        res = _f64(residual)
        lo, hi = shard_range(res.shape[0], world, rank)
        h = res[lo:hi] if h is None else h + res[lo:hi]
    if h is None:
        raise ValueError("nothing to reduce")
    y = layer_norm(h, gamma, beta, eps) if gamma is not None else None
    return h, y


def concat_rows(blocks: Sequence[np.ndarray]) -> np.ndarray:
    """The all-gather along the sequence: the ranks' row blocks stacked in rank order
    ([pwwt] section 5.1, figure 7; rank 0 first as in [typc] section 2.1)."""
    return np.concatenate([_f64(b) for b in blocks], axis=0)


# ----------------------------------------------------------------------------- attention
def split_qkv(Wqkv, hidden: int):
    """The fused QKV weight [H, 3H] read as [Wq | Wk | Wv]."""
    if Wqkv.shape[1] != 3 * hidden:
        raise ValueError("Wqkv must be [H, 3H]")
    return Wqkv[:, :hidden], Wqkv[:, hidden:2 * hidden], Wqkv[:, 2 * hidden:]


def head_range(n_heads: int, world: int, rank: int) -> Tuple[int, int]:
    """Heads owned by a rank: the head dimension split in contiguous blocks ([typc]
    section 3: 64 heads on 4-way TP gives 16 heads per GPU; [pwwt] section 2.2)."""
    return shard_range(n_heads, world, rank)


def _softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, qpos: np.ndarray,
                    causal: bool) -> np.ndarray:
    """One head of one sequence: softmax(q k^T / sqrt(d)) v, where query at position
    qpos[i] sees keys 0..qpos[i] when causal.  Rows are stabilised by their maximum."""
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        kpos = np.arange(k.shape[0])
        s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def attention_heads(Xn, Wqkv, n_heads: int, head_dim: int, rank: int, world: int,
                    batch: int, seq: int, causal: bool = True,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """A_r: outputs of rank r's heads, concatenated in ascending head order.

    Each head h computes softmax(Q_h K_h^T / sqrt(d)) V_h with Q_h = Xn Wq[:, h],
    K_h = Xn Wk[:, h], V_h = Xn Wv[:, h] ([edu] section 1.2.2, formulas 1.8-1.13,
    figure 1.5); heads are independent, so a rank computes its own heads with no
    exchange from the QKV projection to the end of the heads ([pwwt] section 2.2,
    figure 4).  Tokens are laid out [batch * seq] with each sequence contiguous;
    attention never crosses sequences.  ``rows`` selects output tokens; the keys and
    values every selected query needs are always computed in full.
    """
    T, H = Xn.shape
    if T != batch * seq:
        raise ValueError("tokens != batch * seq")
    if n_heads * head_dim != H:
        raise ValueError("hidden != n_heads * head_dim")
    Wq, Wk, Wv = split_qkv(Wqkv, H)
    h0, h1 = head_range(n_heads, world, rank)
    c0, c1 = h0 * head_dim, h1 * head_dim
    rows = np.arange(T) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), c1 - c0), dtype=F64)
    for b in range(batch):
        sel = np.nonzero((rows >= b * seq) & (rows < (b + 1) * seq))[0]
        if len(sel) == 0:
            continue
        qpos = rows[sel] - b * seq
        kend = int(qpos.max()) + 1 if causal else seq
        Xb = Xn[b * seq: b * seq + kend]
        K = matmul(Xb, Wk[:, c0:c1])
        V = matmul(Xb, Wv[:, c0:c1])
        Q = matmul(Xn[rows[sel]], Wq[:, c0:c1])
        for j in range(h1 - h0):
            s = slice(j * head_dim, (j + 1) * head_dim)
            out[sel, s] = _softmax_attend(Q[:, s], K[:, s], V[:, s], qpos, causal)
    return out


def attn_head_shard(Xn, Wqkv, Wo, n_heads: int, head_dim: int, rank: int, world: int,
                    batch: int, seq: int, causal: bool = True,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rank r's attention partial Z_r = A_r . Wo[rows of rank r's heads, :].

    The output projection is row-split over the same head blocks, so each rank's
    contribution is a partial of the full output and the ranks' partials are summed
    ([edu] section 1.2.2, split of W^O into per-head row blocks; [pwwt] section 2.2).
    """
    A = attention_heads(Xn, Wqkv, n_heads, head_dim, rank, world, batch, seq, causal, rows)
    h0, h1 = head_range(n_heads, world, rank)
    return matmul(A, Wo[h0 * head_dim: h1 * head_dim, :])


def attn_head_shard_bf16(Xn, Wqkv, Wo, n_heads: int, head_dim: int, rank: int, world: int,
                         batch: int, seq: int, causal: bool = True,
                         rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rank r's attention partial exchanged in bf16 (as row_linear_partial_bf16): the
    output projection's partial rounded once to bfloat16."""
    return round_bf16(attn_head_shard(Xn, Wqkv, Wo, n_heads, head_dim, rank, world, batch, seq,
                                      causal, rows))


def attn_head_shard_fold(Zsum, Xn, Wqkv, Wo, n_heads: int, head_dim: int, rank: int,
                         world: int, batch: int, seq: int, causal: bool = True,
                         accumulate: bool = True) -> np.ndarray:
    """attn_head_shard with its output projection folded into the running sum Zsum, as
    row_linear_fold does for the row-parallel linear ([pwwt] sections 2.3 and 5.3)."""
    part = attn_head_shard(Xn, Wqkv, Wo, n_heads, head_dim, rank, world, batch, seq, causal)
    if not accumulate:
        return part
    return _f64(Zsum) + part


# ----------------------------------------------------------------------------- MLP, block
def mlp_shard(X, A, B, rank: int, world: int, act: str = "gelu_tanh",
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rank r's MLP partial: act(X . A[:, block r]) . B[block r, :].

    The first linear is column-split and the second row-split, so the column output
    block of rank r is exactly rank r's row input block and only the final partials
    need summing ([typc] section 3; [edu] section 1.2.1, formulas 1.2-1.7, figure
    1.4; [pwwt] section 2.3 figure 5, behaviour as described there).
    """
    Y = col_linear(X, A, rank, world, act, rows)
    k0, k1 = shard_range(B.shape[0], world, rank)
    return matmul(Y, B[k0:k1, :])


def _needed_rows(rows: np.ndarray, batch: int, seq: int, causal: bool) -> np.ndarray:
    need = []
    for b in range(batch):
        sel = rows[(rows >= b * seq) & (rows < (b + 1) * seq)]
        if len(sel):
            end = int(sel.max()) + 1 if causal else (b + 1) * seq
            need.append(np.arange(b * seq, end))
    return np.concatenate(need) if need else np.zeros(0, np.int64)


def block_shard(X, Wqkv, Wo, W1, W2, gamma1, beta1, gamma2, beta2, *, n_heads: int,
                head_dim: int, world: int, batch: int, seq: int, causal: bool = True,
                eps: float = 1e-5, rows: Optional[Sequence[int]] = None,
                keep_partials: bool = True, bf16_partials: bool = False) -> Dict[str, object]:
    """The whole block with every rank's shard, composed as
        Xn = LN(X); h = X + sum_r Attn_r(Xn); hn = LN(h); out = h + sum_r MLP_r(hn)
    ([pwwt] section 2.1 figure 3: LayerNorm, QKV, attention, O, residual add,
    LayerNorm, MLP, residual add, with one all-reduce after O and one after the MLP;
    the residual is the un-normalised input).

    Every step after attention is row-local, so ``rows`` restricts the result to
    those tokens; Xn is computed for the token prefixes their causal keys need.
    bf16_partials: every rank's partial is rounded once to bfloat16 before the sums
    (row_linear_partial_bf16).
    Returns a dict with xn, attn_parts (list over ranks), h, hn, mlp_parts, out.
    """
    T, H = X.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    need = _needed_rows(rows, batch, seq, causal)
    # Xn on the needed tokens (LayerNorm is row-local); other rows are never read.
    Xn = np.zeros((T, H), dtype=F64) if len(need) < T else None
    if Xn is None:
        Xn = layer_norm(X, gamma1, beta1, eps)
    else:
        Xn[need] = layer_norm(X[need], gamma1, beta1, eps)
    rnd = round_bf16 if bf16_partials else (lambda a: a)
    attn_parts = [rnd(attn_head_shard(Xn, Wqkv, Wo, n_heads, head_dim, r, world, batch, seq,
                                      causal, rows)) for r in range(world)]
    h, hn = reduce_residual_layernorm(attn_parts, X[rows], gamma2, beta2, eps)
    mlp_parts = [rnd(mlp_shard(hn, W1, W2, r, world)) for r in range(world)]
    out, _ = reduce_residual_layernorm(mlp_parts, h)
    res = {"rows": rows, "xn": Xn[rows], "h": h, "hn": hn, "out": out}
    if keep_partials:
        res["attn_parts"] = attn_parts
        res["mlp_parts"] = mlp_parts
    return res


def block_forward(X, Wqkv, Wo, W1, W2, gamma1, beta1, gamma2, beta2, *, n_heads: int,
                  head_dim: int, batch: int, seq: int, causal: bool = True,
                  eps: float = 1e-5) -> np.ndarray:
    """The same block on a single device, with no sharding at all: plain multi-head
    attention (all heads, full Wo) and the plain MLP.  The check that a
    tensor-parallel composition equals the single-card computation ([pwwt] section
    3.4 and section 6.2) compares ``block_shard`` against this."""
    T, H = X.shape
    Xn = layer_norm(X, gamma1, beta1, eps)
    A = attention_heads(Xn, Wqkv, n_heads, head_dim, 0, 1, batch, seq, causal)
    h = _f64(X) + matmul(A, Wo)
    hn = layer_norm(h, gamma2, beta2, eps)
    return h + matmul(gelu_tanh(matmul(hn, W1)), W2)
