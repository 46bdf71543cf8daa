"""Pins of the CPU oracle: each ``pin_*`` raises AssertionError when the oracle disagrees
with something the pages or the mathematics fix independently of the oracle itself --
values printed on the pages (tests/golden), closed forms, exact integer identities,
brute force with scalar Python loops on tiny inputs, and library routines (torch CPU,
float64) for the special cases that reduce to them.

The module is imported by test_oracle_pins.py (which runs every pin) and by
test_oracle_mutations.py (which plants mistakes in the oracle and checks that some pin
catches each of them).
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import torch
import torch.nn.functional as TF

import oracle.tp_oracle as O
from workloads.configs import tensor_bytes

GOLDEN = Path(__file__).parent / "golden"


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _ints(rng, shape, lo, hi) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def brute_matmul(A, B) -> np.ndarray:
    """Scalar triple loop (tiny inputs only)."""
    A = np.asarray(A, dtype=np.float64).tolist()
    B = np.asarray(B, dtype=np.float64).tolist()
    n, k, m = len(A), len(B), len(B[0])
    out = [[0.0] * m for _ in range(n)]
    for i in range(n):
        Ai = A[i]
        for j in range(m):
            s = 0.0
            for t in range(k):
                s += Ai[t] * B[t][j]
            out[i][j] = s
    return np.array(out)


def _close(a, b, rtol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _t(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ----------------------------------------------------------------------------- sharding
def pin_shard_golden():
    for line in (GOLDEN / "shard_examples.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        n, world, rank, start, stop = map(int, line.split())
        assert O.shard_range(n, world, rank) == (start, stop), line
        assert O.head_range(n, world, rank) == (start, stop), line


def pin_shard_rejects():
    for args in [(10, 4, 0), (4097, 2, 1), (8, 0, 0), (8, 2, 2), (8, 2, -1)]:
        try:
            O.shard_range(*args)
        except ValueError:
            continue
        raise AssertionError(f"shard_range{args} did not reject")


def pin_shard_tiles_exactly():
    for n, world in [(12, 3), (48, 8), (4096, 4)]:
        seen = []
        for r in range(world):
            a, b = O.shard_range(n, world, r)
            assert b - a == n // world
            seen.extend(range(a, b))
        assert seen == list(range(n))


# ----------------------------------------------------------------------------- linears
def pin_column_concat_bruteforce():
    rng = _rng(11)
    X = rng.standard_normal((3, 5))
    W = rng.standard_normal((5, 8))
    ref = brute_matmul(X, W)
    for world in (1, 2, 4, 8):
        Y = O.concat_columns([O.col_linear(X, W, r, world) for r in range(world)])
        _close(Y, ref, 1e-14, f"column concat world={world}")


def pin_column_concat_integer_exact():
    rng = _rng(12)
    X = _ints(rng, (9, 24), -1, 1)
    W = _ints(rng, (24, 32), -2, 2)
    ref = brute_matmul(X, W)
    for world in (2, 4):
        blocks = [O.col_linear(X, W, r, world) for r in range(world)]
        for r, b in enumerate(blocks):
            c = 32 // world
            assert np.array_equal(b, ref[:, r * c:(r + 1) * c]), f"block {r} of {world}"
        assert np.array_equal(O.concat_columns(blocks), ref)


def pin_row_partials_integer_exact():
    rng = _rng(13)
    X = _ints(rng, (7, 32), -1, 1)
    W = _ints(rng, (32, 12), -2, 2)
    ref = brute_matmul(X, W)
    for world in (1, 2, 4, 8):
        c = 32 // world
        parts = [O.row_linear_partial(X, W, r, world) for r in range(world)]
        for r, p in enumerate(parts):
            assert np.array_equal(p, brute_matmul(X[:, r * c:(r + 1) * c], W[r * c:(r + 1) * c])), \
                f"partial {r} of {world}"
        assert np.array_equal(O.reduce_partials(parts), ref)
        assert np.array_equal(O.reduce_partials(parts[::-1]), ref)


def pin_row_fold_integer_exact():
    """Folding the ranks' partials into one running sum, in ascending rank order, reaches the
    un-split product exactly on integer inputs, and every intermediate running sum is the
    brute-force product over the ranks folded so far.  Rank 0 (no accumulate) ignores
    whatever the running sum held."""
    rng = _rng(31)
    X = _ints(rng, (6, 48), -2, 2)
    W = _ints(rng, (48, 10), -3, 3)
    for world in (1, 2, 3, 4, 8):
        c = 48 // world
        Z = np.full((6, 10), 1e6)
        for r in range(world):
            Z = O.row_linear_fold(Z, X, W, r, world, accumulate=r > 0)
            assert np.array_equal(Z, brute_matmul(X[:, :(r + 1) * c], W[:(r + 1) * c])), \
                f"running sum after rank {r} of {world}"
        assert np.array_equal(Z, brute_matmul(X, W))


def pin_row_partials_float():
    rng = _rng(14)
    X = rng.standard_normal((4, 6))
    W = rng.standard_normal((6, 3))
    parts = [O.row_linear_partial(X, W, r, 3) for r in range(3)]
    _close(O.reduce_partials(parts), brute_matmul(X, W), 1e-14, "row sum")


def pin_rows_subset():
    rng = _rng(15)
    X = rng.standard_normal((10, 8))
    W = rng.standard_normal((8, 6))
    rows = [9, 0, 4]
    _close(O.col_linear(X, W, 1, 2, "gelu_tanh", rows),
           O.col_linear(X, W, 1, 2, "gelu_tanh")[rows], 0, "col rows")
    _close(O.row_linear_partial(X, W, 1, 2, rows), O.row_linear_partial(X, W, 1, 2)[rows],
           0, "row rows")


def pin_power_of_two_scaling_exact():
    rng = _rng(16)
    X = rng.standard_normal((5, 16))
    W = rng.standard_normal((16, 8))
    for r in range(2):
        assert np.array_equal(O.col_linear(4.0 * X, W, r, 2), 4.0 * O.col_linear(X, W, r, 2))
        assert np.array_equal(O.row_linear_partial(X, 0.5 * W, r, 2),
                              0.5 * O.row_linear_partial(X, W, r, 2))


def pin_inner_dim_checked():
    try:
        O.col_linear(np.zeros((2, 3)), np.zeros((4, 4)), 0, 2)
    except ValueError:
        return
    raise AssertionError("mismatched inner dimension accepted")


# ----------------------------------------------------------------------------- GeLU
def pin_gelu_closed_forms():
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    x = np.linspace(-8, 8, 161)
    g = O.gelu_tanh(x)
    # g(x) - g(-x) = x exactly in the mathematics (tanh is odd).
    assert np.max(np.abs((g - O.gelu_tanh(-x)) - x)) < 1e-13
    assert abs(O.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(O.gelu_tanh(np.array([-30.0]))[0]) < 1e-12


def pin_gelu_library():
    x = np.linspace(-10, 10, 2001)
    ref = TF.gelu(_t(x), approximate="tanh").numpy()
    _close(O.gelu_tanh(x), ref, 1e-14, "gelu vs torch tanh-GeLU")


def pin_gelu_approximates_erf_form():
    x = np.linspace(-6, 6, 1201)
    erf_form = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    d = np.abs(O.gelu_tanh(x) - erf_form)
    assert d.max() < 1e-3, "not an approximation of GeLU"
    assert d.max() > 1e-6, "erf form instead of the tanh form"


def pin_column_gelu_library():
    rng = _rng(17)
    X = rng.standard_normal((4, 8))
    W = rng.standard_normal((8, 6))
    ref = TF.gelu(_t(brute_matmul(X, W)), approximate="tanh").numpy()
    Y = O.concat_columns([O.col_linear(X, W, r, 3, "gelu_tanh") for r in range(3)])
    _close(Y, ref, 1e-13, "column + GeLU")


# ----------------------------------------------------------------------------- LayerNorm
def pin_layer_norm_library():
    rng = _rng(18)
    h = 3.0 * rng.standard_normal((6, 33)) + 1.5
    g = 1 + 0.5 * rng.standard_normal(33)
    b = 0.5 * rng.standard_normal(33)
    ref = TF.layer_norm(_t(h), (33,), _t(g), _t(b), eps=1e-5).numpy()
    _close(O.layer_norm(h, g, b, 1e-5), ref, 1e-13, "layer_norm vs torch")


def pin_layer_norm_closed_forms():
    rng = _rng(19)
    b = rng.standard_normal(16)
    y = O.layer_norm(np.full((2, 16), 3.25), np.ones(16), b, 1e-5)
    _close(y, np.broadcast_to(b, (2, 16)), 1e-15, "constant row maps to beta")
    # biased variance: row [0, 2] has mean 1 and variance 1, so eps=0 gives [-1, 1]
    y = O.layer_norm(np.array([[0.0, 2.0]]), eps=0.0)
    _close(y, [[-1.0, 1.0]], 1e-15, "two-element row")
    h = 2.0 * rng.standard_normal((4, 64)) + 0.3
    y = O.layer_norm(h, eps=1e-2)
    var = h.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-13
    _close((y * y).mean(axis=1), var / (var + 1e-2), 1e-13, "mean square")


def pin_reduce_residual_layernorm():
    rng = _rng(20)
    parts = [_ints(rng, (3, 8), -5, 5) for _ in range(4)]
    R = _ints(rng, (3, 8), -3, 3)
    h, y = O.reduce_residual_layernorm(parts, R)
    assert y is None
    assert np.array_equal(h, R + parts[0] + parts[1] + parts[2] + parts[3])
    g = rng.standard_normal(8)
    b = rng.standard_normal(8)
    h, y = O.reduce_residual_layernorm(parts, R, g, b, 1e-5)
    ref = TF.layer_norm(_t(h), (8,), _t(g), _t(b), eps=1e-5).numpy()
    _close(y, ref, 1e-13, "fused LN")
    h0, y0 = O.reduce_residual_layernorm([], R, g, b, 1e-5)
    assert np.array_equal(h0, R)
    _close(y0, TF.layer_norm(_t(R), (8,), _t(g), _t(b), eps=1e-5).numpy(), 1e-13, "plain LN")


def pin_reduce_scatter_integer_exact():
    """Rank r's reduce-scatter block is the ascending-rank sum of row block r of every
    partial (scalar loops), and the blocks stacked in rank order are the full sum."""
    rng = _rng(23)
    P, rows, H = 4, 12, 8
    parts = [_ints(rng, (rows, H), -9, 9) for _ in range(P)]
    blocks = []
    for r in range(P):
        got = O.reduce_scatter_rows(parts, r, P)
        ref = np.zeros((rows // P, H))
        for i in range(rows // P):
            for j in range(H):
                acc = 0.0
                for p in range(P):
                    acc += parts[p][r * (rows // P) + i][j]
                ref[i, j] = acc
        assert np.array_equal(got, ref), r
        blocks.append(got)
    assert np.array_equal(O.concat_rows(blocks), O.reduce_partials(parts))
    for bad in [(10, 4), (12, 5)]:
        try:
            O.reduce_scatter_rows([np.zeros((bad[0], H))] * 2, 0, bad[1])
        except ValueError:
            continue
        raise AssertionError(f"rows={bad[0]} world={bad[1]} not rejected")


def pin_reduce_scatter_layernorm_equals_full():
    """The sequence-parallel epilogue gathered over ranks equals the fused all-reduce
    epilogue: the residual add and LayerNorm act row by row."""
    rng = _rng(24)
    P, rows, H = 4, 16, 24
    parts = [rng.standard_normal((rows, H)) for _ in range(P)]
    R = rng.standard_normal((rows, H))
    g, b = rng.standard_normal(H), rng.standard_normal(H)
    h_full, y_full = O.reduce_residual_layernorm(parts, R, g, b, 1e-5)
    hs, ys = zip(*[O.reduce_scatter_residual_layernorm(parts, R, g, b, 1e-5, r, P)
                   for r in range(P)])
    _close(O.concat_rows(hs), h_full, 1e-15, "gathered h")
    _close(O.concat_rows(ys), y_full, 1e-14, "gathered y")
    lo, hi = O.shard_range(rows, P, 2)
    ref = TF.layer_norm(_t(h_full[lo:hi]), (H,), _t(g), _t(b), eps=1e-5).numpy()
    _close(ys[2], ref, 1e-13, "rank 2 LN")
    lo1, hi1 = O.shard_range(rows, P, 1)
    h0, _ = O.reduce_scatter_residual_layernorm([], R, g, b, 1e-5, 1, P)
    assert np.array_equal(h0, R[lo1:hi1])


# ----------------------------------------------------------------------------- attention
def _attn_inputs(seed, batch, seq, H, scale=0.7):
    rng = _rng(seed)
    Xn = rng.standard_normal((batch * seq, H))
    Wqkv = scale * rng.standard_normal((H, 3 * H)) / math.sqrt(H) * 2.0
    Wo = rng.standard_normal((H, H)) / math.sqrt(H)
    return Xn, Wqkv, Wo


def pin_attention_library_sdpa():
    batch, seq, nh, d = 2, 7, 4, 4
    H = nh * d
    Xn, Wqkv, _ = _attn_inputs(21, batch, seq, H)
    for causal in (True, False):
        A = O.attention_heads(Xn, Wqkv, nh, d, 0, 1, batch, seq, causal)
        x = _t(Xn).reshape(batch, seq, H)
        W = _t(Wqkv)
        q = (x @ W[:, :H]).reshape(batch, seq, nh, d).transpose(1, 2)
        k = (x @ W[:, H:2 * H]).reshape(batch, seq, nh, d).transpose(1, 2)
        v = (x @ W[:, 2 * H:]).reshape(batch, seq, nh, d).transpose(1, 2)
        o = TF.scaled_dot_product_attention(q, k, v, is_causal=causal)
        ref = o.transpose(1, 2).reshape(batch * seq, H).numpy()
        _close(A, ref, 1e-12, f"attention vs SDPA causal={causal}")


def pin_attention_prefix_mean():
    batch, seq, nh, d = 2, 6, 2, 4
    H = nh * d
    Xn, Wqkv, _ = _attn_inputs(22, batch, seq, H)
    Wqkv = Wqkv.copy()
    Wqkv[:, :H] = 0.0  # zero queries: all scores 0, uniform weights over visible keys
    V = brute_matmul(Xn, Wqkv[:, 2 * H:])
    for causal in (True, False):
        A = O.attention_heads(Xn, Wqkv, nh, d, 0, 1, batch, seq, causal)
        ref = np.zeros_like(V)
        for b in range(batch):
            for i in range(seq):
                hi = i + 1 if causal else seq
                ref[b * seq + i] = V[b * seq: b * seq + hi].sum(axis=0) / hi
        _close(A, ref, 1e-14, f"prefix mean causal={causal}")


def pin_attention_first_query():
    batch, seq, nh, d = 3, 5, 2, 4
    H = nh * d
    Xn, Wqkv, _ = _attn_inputs(23, batch, seq, H, scale=3.0)
    A = O.attention_heads(Xn, Wqkv, nh, d, 0, 1, batch, seq, True)
    V = brute_matmul(Xn, Wqkv[:, 2 * H:])
    for b in range(batch):
        _close(A[b * seq], V[b * seq], 1e-14, "first query sees only itself")


def pin_attention_bruteforce():
    batch, seq, nh, d, world = 2, 3, 2, 2, 2
    H = nh * d
    Xn, Wqkv, Wo = _attn_inputs(24, batch, seq, H, scale=2.0)
    Q = brute_matmul(Xn, Wqkv[:, :H])
    K = brute_matmul(Xn, Wqkv[:, H:2 * H])
    V = brute_matmul(Xn, Wqkv[:, 2 * H:])
    for r in range(world):
        A = O.attention_heads(Xn, Wqkv, nh, d, r, world, batch, seq, True)
        Z = O.attn_head_shard(Xn, Wqkv, Wo, nh, d, r, world, batch, seq, True)
        hl = nh // world
        ref = np.zeros((batch * seq, hl * d))
        for b in range(batch):
            for i in range(seq):
                for jh in range(hl):
                    h = r * hl + jh
                    cs = range(h * d, (h + 1) * d)
                    sc = [sum(Q[b * seq + i][c] * K[b * seq + j][c] for c in cs) / math.sqrt(d)
                          for j in range(i + 1)]
                    m = max(sc)
                    w = [math.exp(s - m) for s in sc]
                    tot = sum(w)
                    for c_i, c in enumerate(cs):
                        ref[b * seq + i][jh * d + c_i] = sum(
                            w[j] * V[b * seq + j][c] for j in range(i + 1)) / tot
        _close(A, ref, 1e-13, f"attention brute force rank {r}")
        _close(Z, brute_matmul(ref, Wo[r * hl * d:(r + 1) * hl * d]), 1e-13, f"O partial rank {r}")


def _torch_mha(Xn, Wqkv, Wo, nh, batch, seq, causal):
    """Full multi-head attention with output projection (torch, float64)."""
    H = Xn.shape[1]
    x = _t(Xn).reshape(batch, seq, H).transpose(0, 1)  # [seq, batch, H]
    W = _t(Wqkv)
    mask = None
    if causal:
        mask = torch.triu(torch.ones(seq, seq, dtype=torch.bool), diagonal=1)
    out, _ = TF.multi_head_attention_forward(
        x, x, x, H, nh, None, None, None, None, False, 0.0,
        _t(Wo).T.contiguous(), None, training=False, need_weights=False, attn_mask=mask,
        use_separate_proj_weight=True, q_proj_weight=W[:, :H].T.contiguous(),
        k_proj_weight=W[:, H:2 * H].T.contiguous(), v_proj_weight=W[:, 2 * H:].T.contiguous())
    return out.transpose(0, 1).reshape(batch * seq, H).numpy()


def pin_attention_head_split_equals_mha():
    batch, seq, nh, d = 2, 9, 8, 4
    H = nh * d
    Xn, Wqkv, Wo = _attn_inputs(25, batch, seq, H)
    for causal in (True, False):
        ref = _torch_mha(Xn, Wqkv, Wo, nh, batch, seq, causal)
        for world in (1, 2, 4, 8):
            parts = [O.attn_head_shard(Xn, Wqkv, Wo, nh, d, r, world, batch, seq, causal)
                     for r in range(world)]
            _close(O.reduce_partials(parts), ref, 1e-12, f"head split world={world}")


def pin_attention_fold_equals_mha():
    """The attention shards folded into one running sum in ascending rank order equal
    torch's un-split multi-head attention, for every world size."""
    batch, seq, nh, d = 2, 7, 4, 4
    H = nh * d
    Xn, Wqkv, Wo = _attn_inputs(32, batch, seq, H)
    ref = _torch_mha(Xn, Wqkv, Wo, nh, batch, seq, True)
    for world in (1, 2, 4):
        Z = np.full((batch * seq, H), -3e5)
        for r in range(world):
            Z = O.attn_head_shard_fold(Z, Xn, Wqkv, Wo, nh, d, r, world, batch, seq, True,
                                       accumulate=r > 0)
        _close(Z, ref, 1e-12, f"folded heads world={world}")


def pin_attention_rows_subset():
    batch, seq, nh, d = 2, 11, 4, 4
    H = nh * d
    Xn, Wqkv, Wo = _attn_inputs(26, batch, seq, H)
    rows = [21, 0, 5, 11, 12, 10]
    for causal in (True, False):
        full = O.attn_head_shard(Xn, Wqkv, Wo, nh, d, 1, 2, batch, seq, causal)
        sub = O.attn_head_shard(Xn, Wqkv, Wo, nh, d, 1, 2, batch, seq, causal, rows)
        _close(sub, full[rows], 1e-14, "row subset")


# ----------------------------------------------------------------------------- MLP, block
def pin_mlp_bruteforce():
    rng = _rng(27)
    X = rng.standard_normal((3, 4))
    A = rng.standard_normal((4, 8)) / 2
    B = rng.standard_normal((8, 4)) / 2
    g = TF.gelu(_t(brute_matmul(X, A)), approximate="tanh").numpy()
    ref = brute_matmul(g, B)
    for world in (1, 2, 4):
        Z = O.reduce_partials([O.mlp_shard(X, A, B, r, world) for r in range(world)])
        _close(Z, ref, 1e-13, f"MLP world={world}")


def pin_mlp_equals_single_card():
    rng = _rng(28)
    X = rng.standard_normal((16, 32))
    A = rng.standard_normal((32, 128)) / math.sqrt(32)
    B = rng.standard_normal((128, 32)) / math.sqrt(128)
    ref = (TF.gelu(_t(X) @ _t(A), approximate="tanh") @ _t(B)).numpy()
    for world in (2, 4, 8):
        Z = O.reduce_partials([O.mlp_shard(X, A, B, r, world) for r in range(world)])
        _close(Z, ref, 1e-13, f"MLP single card world={world}")


def _block_inputs(seed, batch, seq, nh, d, F):
    rng = _rng(seed)
    H = nh * d
    X = rng.standard_normal((batch * seq, H))
    Wqkv = rng.standard_normal((H, 3 * H)) / math.sqrt(H)
    Wo = rng.standard_normal((H, H)) / math.sqrt(H)
    W1 = rng.standard_normal((H, F)) / math.sqrt(H)
    W2 = rng.standard_normal((F, H)) / math.sqrt(F)
    g1, b1, g2, b2 = (1 + 0.3 * rng.standard_normal(H), 0.3 * rng.standard_normal(H),
                      1 + 0.3 * rng.standard_normal(H), 0.3 * rng.standard_normal(H))
    return X, Wqkv, Wo, W1, W2, g1, b1, g2, b2


def _torch_block(X, Wqkv, Wo, W1, W2, g1, b1, g2, b2, nh, batch, seq, causal, eps=1e-5):
    H = X.shape[1]
    xn = TF.layer_norm(_t(X), (H,), _t(g1), _t(b1), eps=eps).numpy()
    h = _t(X) + _t(_torch_mha(xn, Wqkv, Wo, nh, batch, seq, causal))
    hn = TF.layer_norm(h, (H,), _t(g2), _t(b2), eps=eps)
    return (h + TF.gelu(hn @ _t(W1), approximate="tanh") @ _t(W2)).numpy()


def pin_block_equals_single_card():
    batch, seq, nh, d, F = 2, 6, 4, 4, 64
    args = _block_inputs(29, batch, seq, nh, d, F)
    ref = _torch_block(*args, nh, batch, seq, True)
    _close(O.block_forward(*args, n_heads=nh, head_dim=d, batch=batch, seq=seq), ref, 1e-12,
           "single-device block")
    for world in (1, 2, 4):
        res = O.block_shard(*args, n_heads=nh, head_dim=d, world=world, batch=batch, seq=seq)
        _close(res["out"], ref, 1e-12, f"block shard world={world}")


def pin_block_rows_subset():
    batch, seq, nh, d, F = 2, 7, 4, 4, 32
    args = _block_inputs(30, batch, seq, nh, d, F)
    full = O.block_shard(*args, n_heads=nh, head_dim=d, world=2, batch=batch, seq=seq)
    rows = [13, 3, 7, 0]
    sub = O.block_shard(*args, n_heads=nh, head_dim=d, world=2, batch=batch, seq=seq, rows=rows)
    for key in ("h", "hn", "out"):
        _close(sub[key], full[key][rows], 1e-14, key)
    for r in range(2):
        _close(sub["attn_parts"][r], full["attn_parts"][r][rows], 1e-14, "attn part")


# ----------------------------------------------------------------------------- backward
def _transpose(M):
    """Explicit transpose by index swapping (no library call)."""
    M = np.asarray(M, np.float64)
    return np.array([[M[i][j] for i in range(M.shape[0])] for j in range(M.shape[1])])


def pin_gelu_grad_closed_forms():
    """gelu'(0) = 1/2; gelu(x) - gelu(-x) = x gives gelu'(x) + gelu'(-x) = 1 exactly; the
    derivative tends to 1 for large x and to 0 for large negative x."""
    assert O.gelu_tanh_grad(np.array([0.0]))[0] == 0.5
    x = np.linspace(-6, 6, 241)
    _close(O.gelu_tanh_grad(x) + O.gelu_tanh_grad(-x), np.ones_like(x), 1e-15, "gelu' symmetry")
    assert abs(O.gelu_tanh_grad(np.array([30.0]))[0] - 1.0) < 1e-15
    assert abs(O.gelu_tanh_grad(np.array([-30.0]))[0]) < 1e-15


def pin_gelu_grad_finite_difference():
    """Central differences of the (separately pinned) gelu_tanh, error O(h^2)."""
    x = np.linspace(-7, 7, 281) + 0.013
    h = 1e-5
    fd = (O.gelu_tanh(x + h) - O.gelu_tanh(x - h)) / (2 * h)
    _close(O.gelu_tanh_grad(x), fd, 1e-9, "gelu' vs central difference")


def pin_gelu_grad_autograd():
    x = torch.linspace(-8, 8, 1601, dtype=torch.float64, requires_grad=True)
    TF.gelu(x, approximate="tanh").sum().backward()
    _close(O.gelu_tanh_grad(x.detach().numpy()), x.grad.numpy(), 1e-14, "gelu' autograd")


def pin_row_backward_integer_exact():
    """Integer inputs: dY_r = dZ . W_r^T and dW_r = Y_r^T . dZ equal scalar-loop products over
    explicitly transposed blocks, exactly, for every rank."""
    rng = _rng(31)
    seq, K, N = 5, 8, 6
    dZ = _ints(rng, (seq, N), -4, 4)
    W = _ints(rng, (K, N), -3, 3)
    for world in (1, 2, 4):
        kl = K // world
        for r in range(world):
            Y = _ints(rng, (seq, kl), -5, 5)
            dY, dW = O.row_linear_backward(dZ, Y, W, r, world)
            Wr = [[W[r * kl + j][n] for n in range(N)] for j in range(kl)]
            assert np.array_equal(dY, brute_matmul(dZ, _transpose(Wr))), f"dY rank {r}/{world}"
            assert np.array_equal(dW, brute_matmul(_transpose(Y), dZ)), f"dW rank {r}/{world}"


def pin_row_backward_activation_factor():
    """With act = gelu_tanh, dY is the plain product times gelu'(U) elementwise (dyadic
    inputs keep the product exact)."""
    rng = _rng(32)
    seq, K, N, world = 4, 8, 5, 2
    dZ = _ints(rng, (seq, N), -4, 4) / 4
    W = _ints(rng, (K, N), -4, 4) / 8
    U = rng.standard_normal((seq, K // world))
    Y = _ints(rng, (seq, K // world), -3, 3)
    for r in range(world):
        plain, _ = O.row_linear_backward(dZ, Y, W, r, world)
        dY, _ = O.row_linear_backward(dZ, Y, W, r, world, U, "gelu_tanh")
        g = np.array([[O.gelu_tanh_grad(np.array([v]))[0] for v in row] for row in U])
        _close(dY, plain * g, 1e-15, "act' factor")


def pin_col_backward_integer_exact():
    """Integer inputs: rank r's dX_part = dU_r . W[:, block r]^T and dW_r = X^T . dU_r by
    scalar loops; the partials summed over ranks equal dU . W^T of the unsplit layer."""
    rng = _rng(33)
    seq, H, N = 5, 6, 8
    X = _ints(rng, (seq, H), -4, 4)
    W = _ints(rng, (H, N), -3, 3)
    dU_full = _ints(rng, (seq, N), -3, 3)
    for world in (1, 2, 4):
        nl = N // world
        parts = []
        for r in range(world):
            dU = dU_full[:, r * nl:(r + 1) * nl]
            dXp, dW = O.col_linear_backward(dU, X, W, r, world)
            Wr = [[W[h][r * nl + j] for j in range(nl)] for h in range(H)]
            assert np.array_equal(dXp, brute_matmul(dU, _transpose(Wr))), f"dX_part {r}/{world}"
            assert np.array_equal(dW, brute_matmul(_transpose(X), dU)), f"dW {r}/{world}"
            parts.append(dXp)
        assert np.array_equal(O.reduce_partials(parts), brute_matmul(dU_full, _transpose(W)))


def _mlp_bwd_inputs(seed, seq, H, F):
    rng = _rng(seed)
    X = rng.standard_normal((seq, H))
    A = rng.standard_normal((H, F)) / math.sqrt(H)
    B = rng.standard_normal((F, H)) / math.sqrt(F)
    dZ = rng.standard_normal((seq, H))
    return X, A, B, dZ


def pin_mlp_backward_autograd():
    """The sharded backward (every rank, partials summed, gradient blocks assembled in rank
    order) equals torch autograd through the unsplit float64 MLP gelu(X A) B."""
    X, A, B, dZ = _mlp_bwd_inputs(34, 6, 8, 32)
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    Z = TF.gelu(tX @ tA, approximate="tanh") @ tB
    (Z * _t(dZ)).sum().backward()
    for world in (1, 2, 4, 8):
        g = O.mlp_backward(X, A, B, dZ, world)
        _close(g["dX"], tX.grad.numpy(), 1e-13, f"dX world={world}")
        _close(g["dA"], tA.grad.numpy(), 1e-13, f"dA world={world}")
        _close(g["dB"], tB.grad.numpy(), 1e-13, f"dB world={world}")


def pin_mlp_backward_finite_difference():
    """Brute force: central differences of the loss sum(dZ * Z), with Z the sum of the
    oracle's forward shard partials, in single entries of X, A and B."""
    X, A, B, dZ = _mlp_bwd_inputs(35, 3, 4, 8)
    world = 2

    def loss(X_, A_, B_):
        Z = O.reduce_partials([O.mlp_shard(X_, A_, B_, r, world) for r in range(world)])
        return float(np.sum(dZ * Z))

    g = O.mlp_backward(X, A, B, dZ, world)
    h = 1e-6
    for name, M, idx in (("X", X, (1, 2)), ("X", X, (2, 0)), ("A", A, (0, 5)), ("A", A, (3, 1)),
                         ("B", B, (6, 3)), ("B", B, (2, 0))):
        Mp, Mm = M.copy(), M.copy()
        Mp[idx] += h
        Mm[idx] -= h
        args_p = {"X": X, "A": A, "B": B}
        args_m = dict(args_p)
        args_p[name], args_m[name] = Mp, Mm
        fd = (loss(args_p["X"], args_p["A"], args_p["B"])
              - loss(args_m["X"], args_m["A"], args_m["B"])) / (2 * h)
        got = g["d" + name][idx]
        assert abs(fd - got) <= 1e-7 * max(1.0, abs(fd)), f"d{name}{idx}: {got} vs {fd}"


# ----------------------------------------------------------------------------- bf16 partials
def pin_round_bf16_closed_forms():
    """Round to nearest, ties to even, at the points where a mistake shows: exact values,
    ties in both directions, the carry into the next binade, overflow, subnormals, zeros."""
    cases = [
        (1.0, 1.0), (1 + 2 ** -7, 1 + 2 ** -7),           # representable
        (1 + 2 ** -8, 1.0),                                # tie -> even (down)
        (1 + 3 * 2 ** -8, 1 + 2 ** -6),                    # tie -> even (up)
        (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7),             # above the tie
        (-(1 + 2 ** -8), -1.0),                            # sign
        (2 - 2 ** -9, 2.0),                                # carries into the next binade
        (257.0, 256.0), (259.0, 260.0), (256.0, 256.0),    # integers: quantum 2 above 256
        ((2 - 2 ** -7) * 2.0 ** 127, (2 - 2 ** -7) * 2.0 ** 127),  # largest finite
        ((2 - 2 ** -8) * 2.0 ** 127, math.inf),            # tie above the largest -> inf
        (2.0 ** -130, 2.0 ** -130),                        # subnormal, representable
        (1.5 * 2.0 ** -133, 2.0 ** -132),                  # subnormal tie -> even
        (2.0 ** -134, 0.0),                                # half the smallest -> 0 (even)
        (0.0, 0.0), (math.inf, math.inf),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = O.round_bf16(x)
    assert np.array_equal(got, want), list(zip(x.tolist(), got.tolist(), want.tolist()))
    assert math.copysign(1.0, O.round_bf16(np.array([-0.0]))[0]) < 0


def pin_round_bf16_library():
    """torch's float32 -> bfloat16 conversion (round to nearest even) on float32 values over
    the whole exponent range: bit-for-bit the same results."""
    rng = _rng(900)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-85, 85, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def pin_row_partial_bf16_integers():
    """Integer partials: exact in bf16 up to 256 in magnitude, rounded to even steps of 2
    between 256 and 512 -- the rounding is applied to each rank's partial, not to the sum."""
    rng = _rng(901)
    X = _ints(rng, (9, 40), -1, 1)
    W = _ints(rng, (40, 16), -2, 2)
    for r in range(2):
        exact = O.row_linear_partial(X, W, r, 2)
        got = O.row_linear_partial_bf16(X, W, r, 2)
        assert np.array_equal(got, exact), "small integer partials are exact in bf16"
    Xb = np.full((1, 4), 64.0)
    Wb = np.array([[1.0], [1.0], [1.0], [1.0 + 1 / 64]])   # partial of rank 0 of 1: 257
    assert O.row_linear_partial(Xb, Wb, 0, 1)[0, 0] == 257.0
    assert O.row_linear_partial_bf16(Xb, Wb, 0, 1)[0, 0] == 256.0
    blk = O.block_shard(*_block_args(), n_heads=2, head_dim=4, world=2, batch=1, seq=3,
                        bf16_partials=True)
    for p in blk["attn_parts"] + blk["mlp_parts"]:
        assert np.array_equal(p, O.round_bf16(p)), "block partials are bf16 values"


def pin_col_backward_bf16_partial():
    """The bf16 input-gradient partial rounds each rank's dU . W_r^T to nearest, ties to even
    (257 -> 256 and 259 -> 260, the two neighbours of a tie in the binade [256, 512)), and
    leaves the weight gradient in full precision."""
    dU = np.ones((1, 3))
    W = np.zeros((2, 6))
    W[0, 3:] = [128.0, 128.0, 1.0]                       # rank 1 of 2: dX_part[0, 0] = 257
    W[1, 3:] = [128.0, 130.0, 1.0]                       #              dX_part[0, 1] = 259
    X = np.array([[0.5, 1.0 + 2.0 ** -12]])
    dXp, dW = O.col_linear_backward(dU, X, W, 1, 2)
    assert dXp.tolist() == [[257.0, 259.0]]
    dXh, dWh = O.col_linear_backward_bf16(dU, X, W, 1, 2)
    assert dXh.tolist() == [[256.0, 260.0]]
    assert np.array_equal(dWh, dW) and dW[1, 0] == 1.0 + 2.0 ** -12, "dW is not rounded"
    rng = _rng(903)
    X, A, B = rng.standard_normal((5, 8)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8))
    dZ = rng.standard_normal((5, 8))
    full = O.mlp_backward(X, A, B, dZ, 2)
    half = O.mlp_backward(X, A, B, dZ, 2, bf16_dx_partials=True)
    parts = [O.mlp_shard_backward(X, A, B, dZ, r, 2, bf16_dx_partials=True)["dX_part"]
             for r in range(2)]
    assert np.array_equal(half["dX"], parts[0] + parts[1])
    assert np.array_equal(half["dA"], full["dA"]) and np.array_equal(half["dB"], full["dB"])
    # two partials, each within 2^-8 (half a bf16 quantum) of its own magnitude
    bound = 2.0 ** -8 * sum(np.abs(O.mlp_shard_backward(X, A, B, dZ, r, 2)["dX_part"])
                            for r in range(2))
    assert np.all(np.abs(half["dX"] - full["dX"]) <= bound)
    assert not np.array_equal(half["dX"], full["dX"])


def _block_args():
    rng = _rng(902)
    H, F = 8, 16
    X = rng.standard_normal((3, H))
    g, b = np.ones(H), np.zeros(H)
    return (X, rng.standard_normal((H, 3 * H)) / 3, rng.standard_normal((H, H)) / 3,
            rng.standard_normal((H, F)) / 3, rng.standard_normal((F, H)) / 4, g, b, g, b)


# ----------------------------------------------------------------------------- accounting
def pin_byte_accounting_golden():
    vals = {}
    for line in (GOLDEN / "byte_accounting.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            vals[k] = int(v)
    one = tensor_bytes(2048, 4096, "bf16")
    assert one == vals["tensor_SH_bf16"]
    assert 2 * one == vals["allreduce_SH_bf16_page_count"]
    assert 4 * one == vals["block_two_allreduces"]


ALL_PINS = {name: fn for name, fn in sorted(globals().items())
            if name.startswith("pin_") and callable(fn)}
