"""ctypes binding of libtp_shard.so: the C entry points under the same names.

Argument marshalling only: torch tensors (or raw integer addresses) become device
pointers, torch streams become hipStream_t handles, and a negative status raises
``TPError``.  Every step of the computation runs in the library's HIP kernels; there is
no other implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from ._build import LIB_PATH

TP_OK = 0
TP_ERR_NULL = -1
TP_ERR_SHAPE = -2
TP_ERR_DIVISIBLE = -3
TP_ERR_RANK = -4
TP_ERR_DTYPE = -5
TP_ERR_ALIGN = -6
TP_ERR_WORKSPACE = -7
TP_ERR_LAUNCH = -8
TP_ERR_SCRATCH = -9
TP_ATTN_SCRATCH_BYTES = 160 << 20

TP_F32 = 0
TP_BF16 = 1
TP_ACT_NONE = 0
TP_ACT_GELU_TANH = 1

EXPORTED = ("tp_col_linear_gelu", "tp_row_linear_partial", "tp_row_linear_fold",
            "tp_col_linear_gelu_save", "tp_row_linear_backward", "tp_col_linear_backward",
            "tp_attn_workspace_bytes", "tp_attn_head_shard", "tp_attn_head_shard_fold",
            "tp_attn_head_shard_noalloc", "tp_partial_reduce_residual_ln",
            "tp_partial_reduce_scatter_residual_ln", "tp_row_linear_partial_bf16",
            "tp_attn_head_shard_bf16", "tp_partial_reduce_residual_ln_bf16",
            "tp_partial_reduce_scatter_residual_ln_bf16", "tp_col_linear_backward_bf16",
            "tp_status_string")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(the HIP library is the only implementation)")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
lib.tp_col_linear_gelu.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _vp]
lib.tp_col_linear_gelu.restype = _int
lib.tp_row_linear_partial.argtypes = [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp]
lib.tp_row_linear_partial.restype = _int
lib.tp_row_linear_fold.argtypes = [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                   _vp]
lib.tp_row_linear_fold.restype = _int
lib.tp_col_linear_gelu_save.argtypes = [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _int,
                                        _int, _int, _vp]
lib.tp_col_linear_gelu_save.restype = _int
lib.tp_row_linear_backward.argtypes = [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64,
                                       _i64, _i64, _int, _int, _int, _int, _int, _vp]
lib.tp_row_linear_backward.restype = _int
lib.tp_col_linear_backward.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                       _int, _int, _int, _int, _vp]
lib.tp_col_linear_backward.restype = _int
lib.tp_col_linear_backward_bf16.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64,
                                            _i64, _int, _int, _int, _vp]
lib.tp_col_linear_backward_bf16.restype = _int
lib.tp_attn_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int, _int, _int]
lib.tp_attn_workspace_bytes.restype = _sz
lib.tp_attn_head_shard.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                   _int, _int, _vp, _sz, _vp]
lib.tp_attn_head_shard.restype = _int
lib.tp_attn_head_shard_fold.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                        _int, _int, _int, _int, _vp, _sz, _vp]
lib.tp_attn_head_shard_fold.restype = _int
lib.tp_attn_head_shard_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                           _int, _int, _int, _vp]
lib.tp_attn_head_shard_noalloc.restype = _int
lib.tp_partial_reduce_residual_ln.argtypes = [_vp, _int, _i64, _vp, _vp, _vp, _f32, _vp, _vp,
                                              _i64, _i64, _int, _vp]
lib.tp_partial_reduce_residual_ln.restype = _int
lib.tp_partial_reduce_scatter_residual_ln.argtypes = [_vp, _int, _i64, _vp, _vp, _vp, _f32, _vp,
                                                      _vp, _i64, _i64, _int, _int, _int, _vp]
lib.tp_partial_reduce_scatter_residual_ln.restype = _int
lib.tp_row_linear_partial_bf16.argtypes = [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                           _vp]
lib.tp_row_linear_partial_bf16.restype = _int
lib.tp_attn_head_shard_bf16.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                        _int, _int, _vp, _sz, _vp]
lib.tp_attn_head_shard_bf16.restype = _int
lib.tp_partial_reduce_residual_ln_bf16.argtypes = [_vp, _int, _i64, _vp, _vp, _vp, _f32, _vp, _vp,
                                                   _i64, _i64, _vp]
lib.tp_partial_reduce_residual_ln_bf16.restype = _int
lib.tp_partial_reduce_scatter_residual_ln_bf16.argtypes = [_vp, _int, _i64, _vp, _vp, _vp, _f32,
                                                           _vp, _vp, _i64, _i64, _int, _int, _vp]
lib.tp_partial_reduce_scatter_residual_ln_bf16.restype = _int
lib.tp_status_string.argtypes = [_int]
lib.tp_status_string.restype = ctypes.c_char_p


class TPError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {tp_status_string(status)} ({status})")


def tp_status_string(status: int) -> str:
    return lib.tp_status_string(int(status)).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int, fn: str) -> int:
    if st != TP_OK:
        raise TPError(st, fn)
    return st


def tp_col_linear_gelu(X, W, Y, ldy: int, seq: int, H: int, N: int, rank: int, world: int,
                       act: int, dtype: int, stream=None) -> int:
    return _check(lib.tp_col_linear_gelu(_ptr(X), _ptr(W), _ptr(Y), ldy, seq, H, N, rank, world,
                                         act, dtype, _stream(stream)), "tp_col_linear_gelu")


def tp_row_linear_partial(X, ldx: int, W, Zpart, seq: int, K: int, N: int, rank: int, world: int,
                          dtype: int, stream=None) -> int:
    return _check(lib.tp_row_linear_partial(_ptr(X), ldx, _ptr(W), _ptr(Zpart), seq, K, N, rank,
                                            world, dtype, _stream(stream)), "tp_row_linear_partial")


def tp_row_linear_fold(X, ldx: int, W, Zsum, seq: int, K: int, N: int, rank: int, world: int,
                       accumulate: int, dtype: int, stream=None) -> int:
    return _check(lib.tp_row_linear_fold(_ptr(X), ldx, _ptr(W), _ptr(Zsum), seq, K, N, rank, world,
                                         int(accumulate), dtype, _stream(stream)),
                  "tp_row_linear_fold")


def tp_col_linear_gelu_save(X, W, Y, ldy: int, U, ldu: int, seq: int, H: int, N: int, rank: int,
                            world: int, dtype: int, stream=None) -> int:
    return _check(lib.tp_col_linear_gelu_save(_ptr(X), _ptr(W), _ptr(Y), ldy, _ptr(U), ldu, seq, H,
                                              N, rank, world, dtype, _stream(stream)),
                  "tp_col_linear_gelu_save")


def tp_row_linear_backward(dZ, W, Y, ldy: int, U, ldu: int, dY, ld_dy: int, dW, ld_dw: int,
                           seq: int, K: int, N: int, rank: int, world: int, act: int,
                           accumulate: int, dtype: int, stream=None) -> int:
    return _check(lib.tp_row_linear_backward(_ptr(dZ), _ptr(W), _ptr(Y), ldy, _ptr(U), ldu,
                                             _ptr(dY), ld_dy, _ptr(dW), ld_dw, seq, K, N, rank,
                                             world, act, int(accumulate), dtype, _stream(stream)),
                  "tp_row_linear_backward")


def tp_col_linear_backward(X, W, dU, ldu: int, dXpart, dW, ld_dw: int, seq: int, H: int, N: int,
                           rank: int, world: int, accumulate: int, dtype: int,
                           stream=None) -> int:
    return _check(lib.tp_col_linear_backward(_ptr(X), _ptr(W), _ptr(dU), ldu, _ptr(dXpart),
                                             _ptr(dW), ld_dw, seq, H, N, rank, world,
                                             int(accumulate), dtype, _stream(stream)),
                  "tp_col_linear_backward")


def tp_col_linear_backward_bf16(X, W, dU, ldu: int, dXpart, dW, ld_dw: int, seq: int, H: int,
                                N: int, rank: int, world: int, accumulate: int,
                                stream=None) -> int:
    return _check(lib.tp_col_linear_backward_bf16(_ptr(X), _ptr(W), _ptr(dU), ldu, _ptr(dXpart),
                                                  _ptr(dW), ld_dw, seq, H, N, rank, world,
                                                  int(accumulate), _stream(stream)),
                  "tp_col_linear_backward_bf16")


def tp_attn_workspace_bytes(batch: int, seq: int, H: int, n_heads: int, head_dim: int, world: int,
                            dtype: int) -> int:
    return int(lib.tp_attn_workspace_bytes(batch, seq, H, n_heads, head_dim, world, dtype))


def tp_attn_head_shard(Xn, Wqkv, Wo, Zpart, batch: int, seq: int, H: int, n_heads: int,
                       head_dim: int, rank: int, world: int, causal: int, dtype: int, workspace,
                       workspace_bytes: int, stream=None) -> int:
    return _check(lib.tp_attn_head_shard(_ptr(Xn), _ptr(Wqkv), _ptr(Wo), _ptr(Zpart), batch, seq,
                                         H, n_heads, head_dim, rank, world, int(causal), dtype,
                                         _ptr(workspace), workspace_bytes, _stream(stream)),
                  "tp_attn_head_shard")


def tp_attn_head_shard_fold(Xn, Wqkv, Wo, Zsum, batch: int, seq: int, H: int, n_heads: int,
                            head_dim: int, rank: int, world: int, causal: int, accumulate: int,
                            dtype: int, workspace, workspace_bytes: int, stream=None) -> int:
    return _check(lib.tp_attn_head_shard_fold(_ptr(Xn), _ptr(Wqkv), _ptr(Wo), _ptr(Zsum), batch,
                                              seq, H, n_heads, head_dim, rank, world, int(causal),
                                              int(accumulate), dtype, _ptr(workspace),
                                              workspace_bytes, _stream(stream)),
                  "tp_attn_head_shard_fold")


def tp_attn_head_shard_noalloc(Xn, Wqkv, Wo, Zpart, batch: int, seq: int, H: int, n_heads: int,
                               head_dim: int, rank: int, world: int, causal: int, dtype: int,
                               stream=None) -> int:
    return _check(lib.tp_attn_head_shard_noalloc(_ptr(Xn), _ptr(Wqkv), _ptr(Wo), _ptr(Zpart),
                                                 batch, seq, H, n_heads, head_dim, rank, world,
                                                 int(causal), dtype, _stream(stream)),
                  "tp_attn_head_shard_noalloc")


def tp_row_linear_partial_bf16(X, ldx: int, W, Zpart, seq: int, K: int, N: int, rank: int,
                               world: int, stream=None) -> int:
    return _check(lib.tp_row_linear_partial_bf16(_ptr(X), ldx, _ptr(W), _ptr(Zpart), seq, K, N,
                                                 rank, world, _stream(stream)),
                  "tp_row_linear_partial_bf16")


def tp_attn_head_shard_bf16(Xn, Wqkv, Wo, Zpart, batch: int, seq: int, H: int, n_heads: int,
                            head_dim: int, rank: int, world: int, causal: int, workspace,
                            workspace_bytes: int, stream=None) -> int:
    return _check(lib.tp_attn_head_shard_bf16(_ptr(Xn), _ptr(Wqkv), _ptr(Wo), _ptr(Zpart), batch,
                                              seq, H, n_heads, head_dim, rank, world, int(causal),
                                              _ptr(workspace), workspace_bytes, _stream(stream)),
                  "tp_attn_head_shard_bf16")


def tp_partial_reduce_residual_ln_bf16(parts, n_parts: int, part_stride: int, residual, gamma,
                                       beta, eps: float, h_out, y_out, rows: int, H: int,
                                       stream=None) -> int:
    return _check(lib.tp_partial_reduce_residual_ln_bf16(_ptr(parts), n_parts, part_stride,
                                                         _ptr(residual), _ptr(gamma), _ptr(beta),
                                                         eps, _ptr(h_out), _ptr(y_out), rows, H,
                                                         _stream(stream)),
                  "tp_partial_reduce_residual_ln_bf16")


def tp_partial_reduce_scatter_residual_ln_bf16(parts, n_parts: int, part_stride: int, residual,
                                               gamma, beta, eps: float, h_out, y_out, rows: int,
                                               H: int, rank: int, world: int,
                                               stream=None) -> int:
    return _check(lib.tp_partial_reduce_scatter_residual_ln_bf16(
        _ptr(parts), n_parts, part_stride, _ptr(residual), _ptr(gamma), _ptr(beta), eps,
        _ptr(h_out), _ptr(y_out), rows, H, rank, world, _stream(stream)),
        "tp_partial_reduce_scatter_residual_ln_bf16")


def tp_partial_reduce_residual_ln(parts, n_parts: int, part_stride: int, residual, gamma, beta,
                                  eps: float, h_out, y_out, rows: int, H: int, dtype: int,
                                  stream=None) -> int:
    return _check(lib.tp_partial_reduce_residual_ln(_ptr(parts), n_parts, part_stride,
                                                    _ptr(residual), _ptr(gamma), _ptr(beta),
                                                    eps, _ptr(h_out), _ptr(y_out), rows, H, dtype,
                                                    _stream(stream)),
                  "tp_partial_reduce_residual_ln")


def tp_partial_reduce_scatter_residual_ln(parts, n_parts: int, part_stride: int, residual, gamma,
                                          beta, eps: float, h_out, y_out, rows: int, H: int,
                                          rank: int, world: int, dtype: int, stream=None) -> int:
    return _check(lib.tp_partial_reduce_scatter_residual_ln(
        _ptr(parts), n_parts, part_stride, _ptr(residual), _ptr(gamma), _ptr(beta), eps,
        _ptr(h_out), _ptr(y_out), rows, H, rank, world, dtype, _stream(stream)),
        "tp_partial_reduce_scatter_residual_ln")
