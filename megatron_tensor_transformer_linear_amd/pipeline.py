"""The simulated tensor-parallel ranks composed from the library calls, on one GPU.

Each class owns the device buffers of one workload and issues the C-ABI calls in the
order the tensor-parallel layer runs them, one rank after another on one stream:

  * the MLP (0539edu.com TP tutorial section 1.2.1; typc.net section 3): per rank, the
    column-parallel linear with GeLU writes its block of the hidden activation into one
    full-width buffer (the all-gather becomes a column offset), then the row-parallel
    linear reads that same block and writes an fp32 partial; the partials are reduced in
    HBM together with the residual add and LayerNorm;
  * the attention-head shard (0539edu.com section 1.2.2; pwwt.cn section 2.2): per rank,
    QKV column split, the rank's heads, O row split to an fp32 partial;
  * the block (pwwt.cn section 2.1, figure 3): LayerNorm, attention shard of every rank,
    reduce + residual + LayerNorm, MLP shard of every rank, reduce + residual.  Here each
    rank's hidden activation is its own dense [T, F/P] buffer, as on separate GPUs.

torch provides device memory and the stream only; all arithmetic is in the HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import tp


def torch_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def tp_dtype(dtype: str) -> int:
    return tp.TP_BF16 if dtype == "bf16" else tp.TP_F32


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Copy a host array to the device: float32 values, or bf16 bit patterns (uint16 or
    int16) reinterpreted as bfloat16."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


class MLPShard:
    """Column-parallel A (GeLU) then row-parallel B, P ranks, then the fused reduce.

    residual_ln=True: h = X + sum_r Z_r and y = LN(h) (io dtype).  Otherwise the partials
    are only summed, into Z (fp32).

    fold=True folds the reduce into the row-parallel products: rank 0 writes one fp32 running
    sum and ranks 1..P-1 add to it in ascending order, so the reduce reads one partial instead
    of P (pwwt.cn sections 2.3, 5.3); the additions are the stacked reduce's, in its order."""

    def __init__(self, X, A, B, world: int, dtype: str, gamma=None, beta=None,
                 eps: float = 1e-5, residual_ln: bool = True, stream=None, fold: bool = False):
        self.X, self.A, self.B = X, A, B
        self.T, self.H = X.shape
        self.F = A.shape[1]
        self.P = world
        self.dt = tp_dtype(dtype)
        self.gamma, self.beta, self.eps = gamma, beta, eps
        self.residual_ln = residual_ln
        self.stream = stream
        self.fold = fold
        dev = X.device
        self.Yfull = torch.empty(self.T, self.F, dtype=torch_dtype(dtype), device=dev)
        # The ranks' fp32 partials, stacked [P, T, H]; with fold, one running sum [1, T, H].
        self.n_parts = 1 if fold else world
        self.parts = torch.empty(self.n_parts, self.T, self.H, dtype=torch.float32, device=dev)
        if residual_ln:
            self.h = torch.empty(self.T, self.H, dtype=torch_dtype(dtype), device=dev)
            self.y = torch.empty_like(self.h)
        else:
            self.Z = torch.empty(self.T, self.H, dtype=torch.float32, device=dev)

    def column(self, r: int):
        fl = self.F // self.P
        tp.tp_col_linear_gelu(self.X, self.A, self.Yfull[:, r * fl:], self.F, self.T, self.H,
                              self.F, r, self.P, tp.TP_ACT_GELU_TANH, self.dt, self.stream)

    def row(self, r: int):
        fl = self.F // self.P
        if self.fold:
            tp.tp_row_linear_fold(self.Yfull[:, r * fl:], self.F, self.B, self.parts[0], self.T,
                                  self.F, self.H, r, self.P, int(r > 0), self.dt, self.stream)
            return
        tp.tp_row_linear_partial(self.Yfull[:, r * fl:], self.F, self.B, self.parts[r], self.T,
                                 self.F, self.H, r, self.P, self.dt, self.stream)

    def reduce(self):
        n = self.T * self.H
        if self.residual_ln:
            tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, n, self.X, self.gamma,
                                             self.beta, self.eps, self.h, self.y, self.T, self.H,
                                             self.dt, self.stream)
        else:
            tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, n, None, None, None, 0.0,
                                             self.Z, None, self.T, self.H, tp.TP_F32, self.stream)

    def step(self):
        for r in range(self.P):
            self.column(r)
            self.row(r)
        self.reduce()


class MLPTrainShard:
    """Forward (keeping the pre-activation) and backward of the tensor-parallel MLP
    Z = sum_r gelu(X . A_r) . B_r in bf16, the P ranks in turn on one GPU.

    Forward of rank r: tp_col_linear_gelu_save writes U_r and Y_r = gelu(U_r) (dense
    [T, F/P] each, as on the rank's own GPU), tp_row_linear_partial its fp32 partial of Z.
    Backward, from the output gradient dZ [T, H] that every rank holds (the forward
    all-reduce is an identity backwards): tp_row_linear_backward gives dU_r (the GeLU's
    derivative fused in) and the rank's row block of dB; tp_col_linear_backward the rank's
    fp32 partial of dX and its column block of dA; reduce_dx sums the partials (the backward
    all-reduce) into dX (bf16).  dA [H, F] and dB [F, H] are fp32, each rank writing its own
    block (the gradient is as sharded as the weight); accumulate=True adds to them.
    bf16_dx_partials=True stores the dX partials in bf16 (tp_col_linear_backward_bf16) and sums
    them with tp_partial_reduce_residual_ln_bf16, halving the exchanged bytes."""

    def __init__(self, X, A, B, dZ, world: int, accumulate: bool = False, stream=None,
                 bf16_dx_partials: bool = False):
        self.X, self.A, self.B, self.dZ = X, A, B, dZ
        self.T, self.H = X.shape
        self.F = A.shape[1]
        self.P = world
        self.fl = self.F // world
        self.accumulate = accumulate
        self.stream = stream
        dev = X.device
        bf = torch.bfloat16
        self.U = torch.empty(world, self.T, self.fl, dtype=bf, device=dev)
        self.Y = torch.empty_like(self.U)
        self.dU = torch.empty_like(self.U)
        self.parts = torch.empty(world, self.T, self.H, dtype=torch.float32, device=dev)
        self.bf16_dx_partials = bf16_dx_partials
        self.dXparts = torch.empty(world, self.T, self.H, device=dev,
                                   dtype=bf if bf16_dx_partials else torch.float32)
        self.dA = torch.zeros(self.H, self.F, dtype=torch.float32, device=dev)
        self.dB = torch.zeros(self.F, self.H, dtype=torch.float32, device=dev)
        self.Z = torch.empty(self.T, self.H, dtype=torch.float32, device=dev)
        self.dX = torch.empty(self.T, self.H, dtype=bf, device=dev)

    def forward_rank(self, r: int):
        tp.tp_col_linear_gelu_save(self.X, self.A, self.Y[r], self.fl, self.U[r], self.fl, self.T,
                                   self.H, self.F, r, self.P, tp.TP_BF16, self.stream)
        tp.tp_row_linear_partial(self.Y[r], self.fl, self.B, self.parts[r], self.T, self.F,
                                 self.H, r, self.P, tp.TP_BF16, self.stream)

    def reduce_z(self):
        tp.tp_partial_reduce_residual_ln(self.parts, self.P, self.T * self.H, None, None, None,
                                         0.0, self.Z, None, self.T, self.H, tp.TP_F32, self.stream)

    def backward_row(self, r: int, input_grad: bool = True, weight_grad: bool = True):
        tp.tp_row_linear_backward(self.dZ, self.B, self.Y[r], self.fl, self.U[r], self.fl,
                                  self.dU[r] if input_grad else None, self.fl,
                                  self.dB[r * self.fl:] if weight_grad else None, self.H, self.T,
                                  self.F, self.H, r, self.P, tp.TP_ACT_GELU_TANH,
                                  int(self.accumulate), tp.TP_BF16, self.stream)

    def backward_col(self, r: int, input_grad: bool = True, weight_grad: bool = True):
        dXp = self.dXparts[r] if input_grad else None
        dA = self.dA[:, r * self.fl:] if weight_grad else None
        if self.bf16_dx_partials:
            tp.tp_col_linear_backward_bf16(self.X, self.A, self.dU[r], self.fl, dXp, dA, self.F,
                                           self.T, self.H, self.F, r, self.P,
                                           int(self.accumulate), self.stream)
        else:
            tp.tp_col_linear_backward(self.X, self.A, self.dU[r], self.fl, dXp, dA, self.F,
                                      self.T, self.H, self.F, r, self.P, int(self.accumulate),
                                      tp.TP_BF16, self.stream)

    def reduce_dx(self):
        if self.bf16_dx_partials:
            tp.tp_partial_reduce_residual_ln_bf16(self.dXparts, self.P, self.T * self.H, None,
                                                  None, None, 0.0, self.dX, None, self.T,
                                                  self.H, self.stream)
        else:
            tp.tp_partial_reduce_residual_ln(self.dXparts, self.P, self.T * self.H, None, None,
                                             None, 0.0, self.dX, None, self.T, self.H,
                                             tp.TP_BF16, self.stream)

    def forward(self):
        for r in range(self.P):
            self.forward_rank(r)
        self.reduce_z()

    def backward(self):
        for r in range(self.P):
            self.backward_row(r)
            self.backward_col(r)
        self.reduce_dx()


class LinearShard:
    """One linear X[T,H].W[H,N]: the column block of chosen ranks, and the row split of
    every rank with the fp32 partial sum Z.

    fold=True folds the reduce into the row-parallel products: rank 0 writes one fp32 running
    sum and ranks 1..P-1 add to it in ascending order, so the reduce reads one partial instead
    of P (pwwt.cn sections 2.3, 5.3); the additions are the stacked reduce's, in its order."""

    def __init__(self, X, W, world: int, dtype: str, col_ranks=(0,), stream=None,
                 fold: bool = False):
        self.X, self.W = X, W
        self.T, self.H = X.shape
        self.N = W.shape[1]
        self.P = world
        self.dt = tp_dtype(dtype)
        self.col_ranks = tuple(col_ranks)
        self.stream = stream
        dev = X.device
        nl = self.N // world
        self.Ycol = {r: torch.empty(self.T, nl, dtype=torch_dtype(dtype), device=dev)
                     for r in self.col_ranks}
        self.fold = fold
        self.n_parts = 1 if fold else world
        self.parts = torch.empty(self.n_parts, self.T, self.N, dtype=torch.float32, device=dev)
        self.Z = torch.empty(self.T, self.N, dtype=torch.float32, device=dev)

    def column(self, r: int, act: int = tp.TP_ACT_NONE):
        Y = self.Ycol[r]
        tp.tp_col_linear_gelu(self.X, self.W, Y, Y.stride(0), self.T, self.H, self.N, r, self.P,
                              act, self.dt, self.stream)

    def row(self, r: int):
        kl = self.H // self.P
        if self.fold:
            tp.tp_row_linear_fold(self.X[:, r * kl:], self.H, self.W, self.parts[0], self.T,
                                  self.H, self.N, r, self.P, int(r > 0), self.dt, self.stream)
            return
        tp.tp_row_linear_partial(self.X[:, r * kl:], self.H, self.W, self.parts[r], self.T,
                                 self.H, self.N, r, self.P, self.dt, self.stream)

    def reduce(self):
        tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, self.T * self.N, None, None,
                                         None, 0.0, self.Z, None, self.T, self.N, tp.TP_F32,
                                         self.stream)

    def step(self):
        for r in self.col_ranks:
            self.column(r)
        for r in range(self.P):
            self.row(r)
        self.reduce()


class AttnShard:
    """The attention-head shard of every rank, and the fp32 sum of their partials.

    fold=True folds the reduce into the row-parallel products: rank 0 writes one fp32 running
    sum and ranks 1..P-1 add to it in ascending order, so the reduce reads one partial instead
    of P (pwwt.cn sections 2.3, 5.3); the additions are the stacked reduce's, in its order."""

    def __init__(self, Xn, Wqkv, Wo, world: int, batch: int, seq: int, n_heads: int,
                 head_dim: int, causal: bool = True, stream=None, fold: bool = False):
        self.Xn, self.Wqkv, self.Wo = Xn, Wqkv, Wo
        self.T, self.H = Xn.shape
        self.P, self.batch, self.seq = world, batch, seq
        self.nh, self.d, self.causal = n_heads, head_dim, causal
        self.stream = stream
        self.fold = fold
        dev = Xn.device
        self.ws_bytes = tp.tp_attn_workspace_bytes(batch, seq, self.H, n_heads, head_dim, world,
                                                   tp.TP_BF16)
        if self.ws_bytes == 0:
            raise ValueError("invalid attention sizes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        # The ranks' fp32 partials, stacked [P, T, H]; with fold, one running sum [1, T, H].
        self.n_parts = 1 if fold else world
        self.parts = torch.empty(self.n_parts, self.T, self.H, dtype=torch.float32, device=dev)
        self.Z = torch.empty(self.T, self.H, dtype=torch.float32, device=dev)

    def workspace_views(self):
        """(QKV_r [T, 3 nb], A_r [T, nb]) bf16 views of the workspace of the last rank run."""
        nb = (self.nh // self.P) * self.d
        n_qkv = self.T * 3 * nb
        flat = self.ws.view(torch.bfloat16)
        return flat[:n_qkv].view(self.T, 3 * nb), flat[n_qkv:n_qkv + self.T * nb].view(self.T, nb)

    def rank(self, r: int, out: Optional[torch.Tensor] = None):
        if self.fold:
            tp.tp_attn_head_shard_fold(self.Xn, self.Wqkv, self.Wo,
                                       self.parts[0] if out is None else out, self.batch,
                                       self.seq, self.H, self.nh, self.d, r, self.P,
                                       int(self.causal), int(r > 0), tp.TP_BF16, self.ws,
                                       self.ws_bytes, self.stream)
            return
        tp.tp_attn_head_shard(self.Xn, self.Wqkv, self.Wo, self.parts[r] if out is None else out,
                              self.batch, self.seq, self.H, self.nh, self.d, r, self.P,
                              int(self.causal), tp.TP_BF16, self.ws, self.ws_bytes, self.stream)

    def reduce(self):
        tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, self.T * self.H, None, None,
                                         None, 0.0, self.Z, None, self.T, self.H, tp.TP_F32,
                                         self.stream)

    def step(self):
        for r in range(self.P):
            self.rank(r)
        self.reduce()


class BlockShard:
    """The whole Transformer block with every rank's attention and MLP shard:
        xn = LN1(X); h = X + sum_r Attn_r(xn); hn = LN2(h); out = h + sum_r MLP_r(hn).

    sequence_parallel=True runs each epilogue as the ranks' reduce-scatters (rank r sums,
    adds the residual to and normalises rows [r T/P, (r+1) T/P)) writing into the full
    buffers at their row offsets, which is the all-gather (pwwt.cn sections 5.1, 5.3).

    fold=True folds the reduce into the row-parallel products: rank 0's output projection
    writes one fp32 [T, H] running sum and ranks 1..P-1 add to it in ascending order, so each
    epilogue reads one partial instead of P (pwwt.cn sections 2.3, 5.3).  The additions are
    the stacked reduce's, in its order, so every output is bit-identical.

    bf16_partials=True stores every rank's partial in bf16, as the pages count the exchanged
    [S, H] partial (pwwt.cn section 5.2: 2 bytes per element): each partial is rounded once
    and the reduces read half the bytes; the sums, residual adds and LayerNorms are the
    fp32-partial path's."""

    def __init__(self, X, Wqkv, Wo, W1, W2, gamma1, beta1, gamma2, beta2, world: int,
                 batch: int, seq: int, n_heads: int, head_dim: int, causal: bool = True,
                 eps: float = 1e-5, stream=None, sequence_parallel: bool = False,
                 fold: bool = False, bf16_partials: bool = False):
        self.X, self.Wqkv, self.Wo, self.W1, self.W2 = X, Wqkv, Wo, W1, W2
        self.g1, self.b1, self.g2, self.b2 = gamma1, beta1, gamma2, beta2
        self.T, self.H = X.shape
        self.F = W1.shape[1]
        self.P, self.batch, self.seq = world, batch, seq
        self.nh, self.d, self.causal, self.eps = n_heads, head_dim, causal, eps
        self.stream = stream
        self.sequence_parallel = sequence_parallel
        self.fold = fold
        self.bf16_partials = bf16_partials
        if bf16_partials and fold:
            raise ValueError("the fold keeps one fp32 running sum: no bf16 partials")
        if sequence_parallel and self.T % world:
            raise ValueError("sequence parallelism needs tokens divisible by the world size")
        dev = X.device
        bf = torch.bfloat16
        self.xn = torch.empty(self.T, self.H, dtype=bf, device=dev)
        self.h = torch.empty_like(self.xn)
        self.hn = torch.empty_like(self.xn)
        self.out = torch.empty_like(self.xn)
        # The hidden activation stays with its rank: Yr[r] = GeLU(hn . W1_r), dense
        # [T, F/P], is the row call's input shard (no gather between the two MLP GEMMs).
        self.Yr = torch.empty(world, self.T, self.F // world, dtype=bf, device=dev)
        # The ranks' fp32 partials, stacked [P, T, H]; with fold, one running sum [1, T, H].
        self.n_parts = 1 if fold else world
        self.parts = torch.empty(self.n_parts, self.T, self.H,
                                 dtype=bf if bf16_partials else torch.float32, device=dev)
        self.ws_bytes = tp.tp_attn_workspace_bytes(batch, seq, self.H, n_heads, head_dim, world,
                                                   tp.TP_BF16)
        if self.ws_bytes == 0:
            raise ValueError("invalid attention sizes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

    def pre_ln(self):
        tp.tp_partial_reduce_residual_ln(None, 0, 0, self.X, self.g1, self.b1, self.eps, None,
                                         self.xn, self.T, self.H, tp.TP_BF16, self.stream)

    def attn(self, r: int):
        if self.fold:
            tp.tp_attn_head_shard_fold(self.xn, self.Wqkv, self.Wo, self.parts[0], self.batch,
                                       self.seq, self.H, self.nh, self.d, r, self.P,
                                       int(self.causal), int(r > 0), tp.TP_BF16, self.ws,
                                       self.ws_bytes, self.stream)
            return
        if self.bf16_partials:
            tp.tp_attn_head_shard_bf16(self.xn, self.Wqkv, self.Wo, self.parts[r], self.batch,
                                       self.seq, self.H, self.nh, self.d, r, self.P,
                                       int(self.causal), self.ws, self.ws_bytes, self.stream)
            return
        tp.tp_attn_head_shard(self.xn, self.Wqkv, self.Wo, self.parts[r], self.batch, self.seq,
                              self.H, self.nh, self.d, r, self.P, int(self.causal), tp.TP_BF16,
                              self.ws, self.ws_bytes, self.stream)

    def _scatter_rows(self, r: int):
        """Rows of rank r's sequence block: (start, count)."""
        n = self.T // self.P
        return r * n, n

    def reduce1(self):
        if self.sequence_parallel:
            for r in range(self.P):
                self.reduce1_scatter(r)
            return
        if self.bf16_partials:
            tp.tp_partial_reduce_residual_ln_bf16(self.parts, self.n_parts, self.T * self.H,
                                                  self.X, self.g2, self.b2, self.eps, self.h,
                                                  self.hn, self.T, self.H, self.stream)
            return
        tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, self.T * self.H, self.X, self.g2,
                                         self.b2, self.eps, self.h, self.hn, self.T, self.H,
                                         tp.TP_BF16, self.stream)

    def reduce1_scatter(self, r: int):
        """Rank r's reduce-scatter + residual + LN2 into its rows of h and hn."""
        a, n = self._scatter_rows(r)
        if self.bf16_partials:
            tp.tp_partial_reduce_scatter_residual_ln_bf16(self.parts, self.n_parts,
                                                          self.T * self.H, self.X, self.g2,
                                                          self.b2, self.eps, self.h[a:a + n],
                                                          self.hn[a:a + n], self.T, self.H, r,
                                                          self.P, self.stream)
            return
        tp.tp_partial_reduce_scatter_residual_ln(self.parts, self.n_parts, self.T * self.H, self.X,
                                                 self.g2, self.b2, self.eps, self.h[a:a + n],
                                                 self.hn[a:a + n], self.T, self.H, r, self.P,
                                                 tp.TP_BF16, self.stream)

    def mlp_col(self, r: int):
        fl = self.F // self.P
        tp.tp_col_linear_gelu(self.hn, self.W1, self.Yr[r], fl, self.T, self.H, self.F, r,
                              self.P, tp.TP_ACT_GELU_TANH, tp.TP_BF16, self.stream)

    def mlp_row(self, r: int):
        fl = self.F // self.P
        if self.fold:
            tp.tp_row_linear_fold(self.Yr[r], fl, self.W2, self.parts[0], self.T, self.F, self.H,
                                  r, self.P, int(r > 0), tp.TP_BF16, self.stream)
            return
        if self.bf16_partials:
            tp.tp_row_linear_partial_bf16(self.Yr[r], fl, self.W2, self.parts[r], self.T, self.F,
                                          self.H, r, self.P, self.stream)
            return
        tp.tp_row_linear_partial(self.Yr[r], fl, self.W2, self.parts[r], self.T, self.F, self.H,
                                 r, self.P, tp.TP_BF16, self.stream)

    def reduce2(self):
        if self.sequence_parallel:
            for r in range(self.P):
                self.reduce2_scatter(r)
            return
        if self.bf16_partials:
            tp.tp_partial_reduce_residual_ln_bf16(self.parts, self.n_parts, self.T * self.H,
                                                  self.h, None, None, 0.0, self.out, None, self.T,
                                                  self.H, self.stream)
            return
        tp.tp_partial_reduce_residual_ln(self.parts, self.n_parts, self.T * self.H, self.h, None,
                                         None, 0.0, self.out, None, self.T, self.H, tp.TP_BF16,
                                         self.stream)

    def reduce2_scatter(self, r: int):
        """Rank r's reduce-scatter + residual into its rows of out."""
        a, n = self._scatter_rows(r)
        if self.bf16_partials:
            tp.tp_partial_reduce_scatter_residual_ln_bf16(self.parts, self.n_parts,
                                                          self.T * self.H, self.h, None, None,
                                                          0.0, self.out[a:a + n], None, self.T,
                                                          self.H, r, self.P, self.stream)
            return
        tp.tp_partial_reduce_scatter_residual_ln(self.parts, self.n_parts, self.T * self.H, self.h,
                                                 None, None, 0.0, self.out[a:a + n], None,
                                                 self.T, self.H, r, self.P, tp.TP_BF16,
                                                 self.stream)

    def attention_phase(self):
        self.pre_ln()
        for r in range(self.P):
            self.attn(r)

    def mlp_phase(self):
        # Every rank's column product, then every rank's row product: the ranks are
        # independent and each keeps its hidden block in its own buffer, so the order changes
        # no result (the folded row products still add in ascending rank order).
        for r in range(self.P):
            self.mlp_col(r)
        for r in range(self.P):
            self.mlp_row(r)

    def step(self):
        self.attention_phase()
        self.reduce1()
        self.mlp_phase()
        self.reduce2()
