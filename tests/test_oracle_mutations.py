"""Plant plausible mistakes in the CPU oracle (on the CPU only) and check that at least
one pin catches each.  This is the evidence that the pins are sharp enough to trust the
oracle: a dropped term, a wrong sign or index, a transposed operand, a reversed rank order
or a wrong constant must all be visible."""
import math

import numpy as np
import pytest

import oracle.tp_oracle as O
from oracle_pins import ALL_PINS

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _shard_off_by_one(n, world, rank):
    a, b = _orig["shard_range"](n, world, rank)
    return (a + 1, b + 1) if rank + 1 < world else (a, b)


def _shard_reversed(n, world, rank):
    return _orig["shard_range"](n, world, world - 1 - rank)


def _shard_floor(n, world, rank):
    if world < 1 or not 0 <= rank < world:
        raise ValueError
    c = n // world
    return rank * c, (rank + 1) * c


def _gelu_const(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.44715 * x ** 3)))


def _gelu_erf(x):
    x = np.asarray(x, np.float64)
    return np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x.ravel()]).reshape(x.shape)


def _gelu_swapped_sqrt(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(math.pi / 2.0) * (x + 0.044715 * x ** 3)))


def _ln_unbiased(h, gamma=None, beta=None, eps=1e-5):
    h = np.asarray(h, np.float64)
    mu = h.mean(axis=-1, keepdims=True)
    var = h.var(axis=-1, ddof=1, keepdims=True)
    y = (h - mu) / np.sqrt(var + eps)
    y = y * gamma if gamma is not None else y
    return y + beta if beta is not None else y


def _ln_no_eps(h, gamma=None, beta=None, eps=1e-5):
    return _orig["layer_norm"](h, gamma, beta, 0.0)


def _ln_swapped_affine(h, gamma=None, beta=None, eps=1e-5):
    return _orig["layer_norm"](h, beta, gamma, eps)


def _attend_no_scale(q, k, v, qpos, causal):
    return _orig["_softmax_attend"](q * math.sqrt(q.shape[1]), k, v, qpos, causal)


def _attend_strict_mask(q, k, v, qpos, causal):
    s = (q @ k.T) / math.sqrt(q.shape[1])
    if causal:
        kpos = np.arange(k.shape[0])
        s = np.where(kpos[None, :] < qpos[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v


def _attend_wrong_axis(q, k, v, qpos, causal):
    s = (q @ k.T) / math.sqrt(q.shape[1])
    if causal:
        kpos = np.arange(k.shape[0])
        s = np.where(kpos[None, :] <= qpos[:, None], s, -1e300)
    p = np.exp(s - s.max(axis=0, keepdims=True))
    return (p / p.sum(axis=0, keepdims=True)) @ v


def _split_qkv_kv_swapped(Wqkv, hidden):
    q, k, v = _orig["split_qkv"](Wqkv, hidden)
    return q, v, k


def _reduce_drop_last(parts):
    return _orig["reduce_partials"](parts[:-1]) if len(parts) > 1 else _orig["reduce_partials"](parts)


def _concat_reversed(blocks):
    return _orig["concat_columns"](list(blocks)[::-1])


def _col_split_rows(X, W, rank, world, act="none", rows=None):
    k0, k1 = _orig["shard_range"](W.shape[0], world, rank)
    Xs = X if rows is None else X[np.asarray(rows)]
    return _orig["_act"](_orig["matmul"](Xs[:, k0:k1], W[k0:k1, :]), act)


def _row_first_block_of_x(X, W, rank, world, rows=None):
    k0, k1 = _orig["shard_range"](W.shape[0], world, rank)
    Xs = X if rows is None else X[np.asarray(rows)]
    return _orig["matmul"](Xs[:, : k1 - k0], W[k0:k1, :])


def _mlp_block0_of_b(X, A, B, rank, world, act="gelu_tanh", rows=None):
    Y = _orig["col_linear"](X, A, rank, world, act, rows)
    k0, k1 = _orig["shard_range"](B.shape[0], world, 0)
    return _orig["matmul"](Y, B[k0:k1, :])


def _attn_wo_columns(Xn, Wqkv, Wo, n_heads, head_dim, rank, world, batch, seq, causal=True,
                     rows=None):
    A = _orig["attention_heads"](Xn, Wqkv, n_heads, head_dim, rank, world, batch, seq, causal, rows)
    h0, h1 = _orig["head_range"](n_heads, world, rank)
    return _orig["matmul"](A, Wo[:, h0 * head_dim: h1 * head_dim].T)


def _residual_added_twice(parts, residual=None, gamma=None, beta=None, eps=1e-5):
    h, y = _orig["reduce_residual_layernorm"](parts, residual, gamma, beta, eps)
    if residual is not None and len(parts):
        h = h + np.asarray(residual, np.float64)
    return h, y


def _scatter_rank0_block(parts, rank, world):
    return _orig["reduce_scatter_rows"](parts, 0, world)


def _scatter_residual_unsliced(parts, residual, gamma, beta, eps, rank, world):
    h = _orig["reduce_scatter_rows"](parts, rank, world) if len(parts) else None
    res = np.asarray(residual, np.float64)[: (h.shape[0] if h is not None else residual.shape[0] // world)]
    h = res if h is None else h + res
    return h, (_orig["layer_norm"](h, gamma, beta, eps) if gamma is not None else None)


def _gather_rows_reversed(blocks):
    return _orig["concat_rows"](list(blocks)[::-1])


def _gelu_grad_first_term_only(x):
    x = np.asarray(x, np.float64)
    return 0.5 * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def _gelu_grad_minus(x):
    x = np.asarray(x, np.float64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (x + 0.044715 * x ** 3))
    return 0.5 * (1.0 + t) - 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x)


def _gelu_grad_no_three(x):
    x = np.asarray(x, np.float64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (x + 0.044715 * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 0.044715 * x * x)


def _row_bwd_no_act(dZ, Y, W, rank, world, U=None, act="none"):
    return _orig["row_linear_backward"](dZ, Y, W, rank, world)


def _row_bwd_act_of_output(dZ, Y, W, rank, world, U=None, act="none"):
    return _orig["row_linear_backward"](dZ, Y, W, rank, world, Y, act)


def _row_bwd_rank0_block(dZ, Y, W, rank, world, U=None, act="none"):
    return _orig["row_linear_backward"](dZ, Y, W, 0, world, U, act)


def _row_bwd_wgrad_transposed(dZ, Y, W, rank, world, U=None, act="none"):
    dY, dW = _orig["row_linear_backward"](dZ, Y, W, rank, world, U, act)
    return dY, np.asarray(dZ, np.float64).T @ np.asarray(Y, np.float64)


def _col_bwd_rank0_block(dU, X, W, rank, world):
    return _orig["col_linear_backward"](dU, X, W, 0, world)


def _col_bwd_wgrad_uses_x_block(dU, X, W, rank, world):
    dXp, _ = _orig["col_linear_backward"](dU, X, W, rank, world)
    X = np.asarray(X, np.float64)
    n = np.asarray(dU).shape[1]
    return dXp, X[:, :n].T @ np.asarray(dU, np.float64) if X.shape[1] >= n else X.T @ dU


def _fold_ignores_running_sum(Zsum, X, W, rank, world, accumulate):
    return _orig["row_linear_fold"](Zsum, X, W, rank, world, False)


def _fold_always_accumulates(Zsum, X, W, rank, world, accumulate):
    return _orig["row_linear_fold"](Zsum, X, W, rank, world, True)


def _attn_fold_ignores_running_sum(Zsum, *args, accumulate=True, **kw):
    return _orig["attn_head_shard_fold"](Zsum, *args, accumulate=False, **kw)


def _bf16_half_away(x):
    x = np.asarray(x, np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    out[fin] = np.sign(x[fin]) * np.floor(np.abs(x[fin]) / q + 0.5) * q
    return out


def _bf16_truncate(x):
    x = np.asarray(x, np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    out[fin] = np.trunc(x[fin] / q) * q
    return out


def _bf16_seven_bits(x):
    x = np.asarray(x, np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 6)
    out[fin] = np.rint(x[fin] / q) * q
    return out


def _row_partial_bf16_unrounded(X, W, rank, world, rows=None):
    return _orig["row_linear_partial"](X, W, rank, world, rows)


def _col_bwd_bf16_unrounded(dU, X, W, rank, world):
    return _orig["col_linear_backward"](dU, X, W, rank, world)


def _col_bwd_bf16_rounds_weight_grad(dU, X, W, rank, world):
    dXp, dW = _orig["col_linear_backward"](dU, X, W, rank, world)
    return _orig["round_bf16"](dXp), _orig["round_bf16"](dW)


MUTATIONS = {
    "bf16_round_half_away": ("round_bf16", _bf16_half_away),
    "bf16_truncate": ("round_bf16", _bf16_truncate),
    "bf16_seven_significant_bits": ("round_bf16", _bf16_seven_bits),
    "row_partial_bf16_unrounded": ("row_linear_partial_bf16", _row_partial_bf16_unrounded),
    "col_bwd_bf16_unrounded": ("col_linear_backward_bf16", _col_bwd_bf16_unrounded),
    "col_bwd_bf16_rounds_weight_grad": ("col_linear_backward_bf16",
                                        _col_bwd_bf16_rounds_weight_grad),
    "shard_off_by_one": ("shard_range", _shard_off_by_one),
    "shard_reversed_ranks": ("shard_range", _shard_reversed),
    "shard_floor_remainder": ("shard_range", _shard_floor),
    "gelu_wrong_cubic_constant": ("gelu_tanh", _gelu_const),
    "gelu_erf_form": ("gelu_tanh", _gelu_erf),
    "gelu_inverted_sqrt": ("gelu_tanh", _gelu_swapped_sqrt),
    "layernorm_unbiased_variance": ("layer_norm", _ln_unbiased),
    "layernorm_missing_eps": ("layer_norm", _ln_no_eps),
    "layernorm_gamma_beta_swapped": ("layer_norm", _ln_swapped_affine),
    "attention_missing_scale": ("_softmax_attend", _attend_no_scale),
    "attention_strict_causal_mask": ("_softmax_attend", _attend_strict_mask),
    "attention_softmax_wrong_axis": ("_softmax_attend", _attend_wrong_axis),
    "qkv_k_v_swapped": ("split_qkv", _split_qkv_kv_swapped),
    "reduce_drops_last_rank": ("reduce_partials", _reduce_drop_last),
    "gather_reversed_rank_order": ("concat_columns", _concat_reversed),
    "column_split_on_rows": ("col_linear", _col_split_rows),
    "row_split_reads_first_x_block": ("row_linear_partial", _row_first_block_of_x),
    "mlp_wrong_b_block": ("mlp_shard", _mlp_block0_of_b),
    "o_projection_transposed": ("attn_head_shard", _attn_wo_columns),
    "residual_added_twice": ("reduce_residual_layernorm", _residual_added_twice),
    "scatter_takes_rank0_rows": ("reduce_scatter_rows", _scatter_rank0_block),
    "scatter_residual_not_sliced": ("reduce_scatter_residual_layernorm", _scatter_residual_unsliced),
    "gather_rows_reversed": ("concat_rows", _gather_rows_reversed),
    "gelu_grad_first_term_only": ("gelu_tanh_grad", _gelu_grad_first_term_only),
    "gelu_grad_wrong_sign": ("gelu_tanh_grad", _gelu_grad_minus),
    "gelu_grad_missing_three": ("gelu_tanh_grad", _gelu_grad_no_three),
    "row_bwd_drops_act_factor": ("row_linear_backward", _row_bwd_no_act),
    "row_bwd_act_at_output": ("row_linear_backward", _row_bwd_act_of_output),
    "row_bwd_rank0_weight_block": ("row_linear_backward", _row_bwd_rank0_block),
    "row_bwd_weight_grad_transposed": ("row_linear_backward", _row_bwd_wgrad_transposed),
    "col_bwd_rank0_weight_block": ("col_linear_backward", _col_bwd_rank0_block),
    "col_bwd_weight_grad_x_block": ("col_linear_backward", _col_bwd_wgrad_uses_x_block),
    "fold_ignores_running_sum": ("row_linear_fold", _fold_ignores_running_sum),
    "fold_accumulates_on_rank0": ("row_linear_fold", _fold_always_accumulates),
    "attn_fold_ignores_running_sum": ("attn_head_shard_fold", _attn_fold_ignores_running_sum),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_is_caught(mutation, monkeypatch):
    target, fn = MUTATIONS[mutation]
    monkeypatch.setattr(O, target, fn)
    caught = []
    for name, pin in ALL_PINS.items():
        try:
            pin()
        except Exception as e:  # an assertion, or the mutated oracle crashing
            caught.append(f"{name}: {type(e).__name__}")
    assert caught, f"no pin catches mutation {mutation}"


def test_unmutated_oracle_passes_every_pin():
    for name, pin in ALL_PINS.items():
        pin()
