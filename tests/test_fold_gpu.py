"""GPU parity of the folded reduce: the row-parallel products add their partials into one
fp32 running sum in ascending rank order (tp_row_linear_fold, tp_attn_head_shard_fold)
instead of stacking them for the reduce kernel.

The folded sum performs the stacked reduce's additions in the same order, so every result
must be bit-identical to the stacked path, which the parity tests check against the oracle;
each case is also checked against the oracle's folded sum directly."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
from gpu_helpers import check, check_exact, dev, dev_values, host, say
from workloads import generate, get_config
from workloads.configs import small_variant
from workloads.synth import integer_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(gpu):
    from megatron_tensor_transformer_linear_amd import pipeline, tp
    torch.cuda.set_device(0)
    return tp, pipeline


def _sync():
    torch.cuda.synchronize()


def _same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    assert a.shape == b.shape, what
    same = torch.eq(a.contiguous().view(view), b.contiguous().view(view))
    bad = int((~same).sum())
    assert bad == 0, f"{what}: {bad} of {a.numel()} elements differ from the stacked path"


def _qkv_values(t):
    return np.hstack([t["Wq"].values(), t["Wk"].values(), t["Wv"].values()])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("world", [1, 2, 4, 8])
def test_row_fold_integer_exact(lib, dtype, world):
    """Integer X in {-1,0,1} and W in {-2..2}: every running sum is an exact integer below
    2^24, so after each rank it must equal the oracle's running sum bit for bit."""
    tp, pl = lib
    T, K, N = 260, 1152, 392
    rng = np.random.Generator(np.random.PCG64(300 + world))
    X = integer_matrix(rng, (T, K), -1, 1, dtype)
    W = integer_matrix(rng, (K, N), -2, 2, dtype)
    Xd, Wd = dev(X), dev(W)
    Z = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    ref = None
    kl = K // world
    for r in range(world):
        say(f"  row fold integer dtype={dtype} world={world} rank={r}")
        tp.tp_row_linear_fold(Xd[:, r * kl:], K, Wd, Z, T, K, N, r, world, int(r > 0),
                              pl.tp_dtype(dtype))
        _sync()
        ref = O.row_linear_fold(ref, X.values(), W.values(), r, world, r > 0)
        check_exact(f"running sum after rank {r}", Z, ref, "f32")
    check_exact("folded sum = X.W", Z, O.matmul(X.values(), W.values()), "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_accumulates_onto_existing_sum(lib, dtype):
    """accumulate != 0 adds to whatever the buffer holds (here a prefilled integer matrix);
    accumulate == 0 ignores it (here NaN)."""
    tp, pl = lib
    T, K, N, world = 136, 512, 264, 4
    rng = np.random.Generator(np.random.PCG64(310))
    X = integer_matrix(rng, (T, K), -1, 1, dtype)
    W = integer_matrix(rng, (K, N), -2, 2, dtype)
    C = rng.integers(-50, 51, size=(T, N)).astype(np.float64)
    Xd, Wd = dev(X), dev(W)
    kl = K // world
    for r in (0, 3):
        say(f"  fold onto existing sum dtype={dtype} rank={r}")
        Z = torch.tensor(C, dtype=torch.float32, device="cuda")
        tp.tp_row_linear_fold(Xd[:, r * kl:], K, Wd, Z, T, K, N, r, world, 1, pl.tp_dtype(dtype))
        _sync()
        part = O.row_linear_partial(X.values(), W.values(), r, world)
        check_exact(f"C + partial rank {r}", Z, O.row_linear_fold(C, X.values(), W.values(), r,
                                                                 world, True), "f32")
        Z.fill_(float("nan"))
        tp.tp_row_linear_fold(Xd[:, r * kl:], K, Wd, Z, T, K, N, r, world, 0, pl.tp_dtype(dtype))
        _sync()
        check_exact(f"partial rank {r} over NaN", Z, part, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N,world", [(300, 1088, 392, 2), (70, 2048, 264, 8),
                                         (513, 4096, 1000, 4)])
def test_linear_fold_bit_identical(lib, dtype, T, K, N, world):
    """Gaussian inputs with ragged tiles: the folded sum has the stacked reduce's bits."""
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(320 + world))
    Xd = dev_values(rng.standard_normal((T, K)).astype(np.float32), dtype)
    Wd = dev_values((rng.standard_normal((K, N)) / np.sqrt(K)).astype(np.float32), dtype)
    Xv, Wv = host(Xd), host(Wd)
    stacked = pl.LinearShard(Xd, Wd, world, dtype, col_ranks=())
    folded = pl.LinearShard(Xd, Wd, world, dtype, col_ranks=(), fold=True)
    say(f"  linear fold vs stacked dtype={dtype} T={T} K={K} N={N} world={world}")
    stacked.step()
    folded.step()
    _sync()
    _same_bits(folded.parts[0], stacked.Z, "folded running sum")
    _same_bits(folded.Z, stacked.Z, "Z")
    ref = None
    for r in range(world):
        ref = O.row_linear_fold(ref, Xv, Wv, r, world, r > 0)
    check("folded sum vs oracle", folded.Z, ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mlp_fold_bit_identical(lib, dtype):
    tp, pl = lib
    cfg = small_variant("mlp_f32_tp2" if dtype == "f32" else "mlp_bf16_tp4")
    t = generate(cfg)
    kw = {} if dtype == "f32" else dict(gamma=dev(t["gamma"]), beta=dev(t["beta"]), eps=cfg.eps)
    kw["residual_ln"] = dtype != "f32"
    args = (dev(t["X"]), dev(t["A"]), dev(t["B"]), cfg.world, dtype)
    stacked = pl.MLPShard(*args, **kw)
    folded = pl.MLPShard(*args, fold=True, **kw)
    say(f"  MLP fold vs stacked {cfg}")
    stacked.step()
    folded.step()
    _sync()
    names = ("Z",) if dtype == "f32" else ("h", "y")
    for name in names:
        _same_bits(getattr(folded, name), getattr(stacked, name), name)
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    ref = O.reduce_partials([O.mlp_shard(X, A, B, r, cfg.world) for r in range(cfg.world)])
    if dtype == "f32":
        check("Z vs oracle", folded.Z, ref, "f32")
    else:
        h, y = O.reduce_residual_layernorm([ref], X, t["gamma"].values(), t["beta"].values(),
                                           cfg.eps)
        check("h vs oracle", folded.h, h, "bf16")
        check("y vs oracle", folded.y, y, "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_attention_fold_bit_identical(lib, causal):
    tp, pl = lib
    cfg = small_variant("attn_bf16_tp4").with_(causal=causal)
    t = generate(cfg)
    Xn, Wqkv, Wo = t["X"].values(), _qkv_values(t), t["Wo"].values()
    args = (dev(t["X"]), dev_values(Wqkv, "bf16"), dev(t["Wo"]), cfg.world, cfg.batch, cfg.seq,
            cfg.n_heads, cfg.head_dim, causal)
    stacked = pl.AttnShard(*args)
    folded = pl.AttnShard(*args, fold=True)
    say(f"  attention fold vs stacked causal={causal} {cfg}")
    stacked.step()
    folded.step()
    _sync()
    _same_bits(folded.parts[0], stacked.Z, "folded running sum")
    _same_bits(folded.Z, stacked.Z, "Z")
    ref = None
    for r in range(cfg.world):
        ref = O.attn_head_shard_fold(ref, Xn, Wqkv, Wo, cfg.n_heads, cfg.head_dim, r, cfg.world,
                                     cfg.batch, cfg.seq, causal, accumulate=r > 0)
    check("folded sum vs oracle", folded.Z, ref, "bf16")


def _block(pl, cfg, t, **kw):
    return pl.BlockShard(dev(t["X"]), dev_values(_qkv_values(t), "bf16"), dev(t["Wo"]),
                         dev(t["W1"]), dev(t["W2"]), dev(t["gamma"]), dev(t["beta"]),
                         dev(t["gamma"]), dev(t["beta"]), cfg.world, cfg.batch, cfg.seq,
                         cfg.n_heads, cfg.head_dim, cfg.causal, cfg.eps, **kw)


@pytest.mark.parametrize("sequence_parallel", [False, True])
def test_block_fold_bit_identical(lib, sequence_parallel):
    tp, pl = lib
    cfg = small_variant("block_bf16_tp8")
    t = generate(cfg)
    stacked = _block(pl, cfg, t)
    folded = _block(pl, cfg, t, fold=True, sequence_parallel=sequence_parallel)
    say(f"  block fold (sequence_parallel={sequence_parallel}) vs stacked {cfg}")
    stacked.step()
    folded.step()
    _sync()
    for name in ("xn", "h", "hn", "out"):
        _same_bits(getattr(folded, name), getattr(stacked, name), name)
    g, b = t["gamma"].values(), t["beta"].values()
    ref = O.block_shard(t["X"].values(), _qkv_values(t), t["Wo"].values(), t["W1"].values(),
                        t["W2"].values(), g, b, g, b, n_heads=cfg.n_heads,
                        head_dim=cfg.head_dim, world=cfg.world, batch=cfg.batch, seq=cfg.seq,
                        causal=cfg.causal, eps=cfg.eps)
    check("out vs oracle", folded.out, ref["out"], "bf16")


@pytest.mark.timeout(600)
def test_full_block_fold_bit_identical(lib):
    """The full-size block, launched as the bench launches it: folded and stacked epilogues
    give the same bits in every output (the stacked path is checked against the oracle on
    sampled rows by the block parity test)."""
    tp, pl = lib
    cfg = get_config("block_bf16_tp8")
    t = generate(cfg)
    say(f"  full block fold vs stacked {cfg.name}: inputs generated")
    stacked = _block(pl, cfg, t)
    stacked.step()
    _sync()
    outs = {name: getattr(stacked, name).clone() for name in ("h", "hn", "out")}
    del stacked
    torch.cuda.empty_cache()
    folded = _block(pl, cfg, t, fold=True)
    folded.step()
    _sync()
    say("  full block fold: comparing")
    for name, ref in outs.items():
        _same_bits(getattr(folded, name), ref, name)
