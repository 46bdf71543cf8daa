"""GPU parity: the HIP library (through its C ABI) against the float64 CPU oracle.

Bit-exact where the result is exact in both (shard extraction, concatenation, integer
GEMMs); otherwise the tolerance rule of gpu_helpers.check.  Reduced-size variants of the
five workloads (several tiles plus ragged tails) are compared element by element; the
full-size workloads, launched exactly as the bench launches them, on every element."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
from gpu_helpers import check, check_exact, dev, dev_values, host, sample_rows, say
from workloads import generate, get_config
from workloads.configs import small_variant
from workloads.synth import from_values, integer_matrix, random_affine

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(gpu):
    from megatron_tensor_transformer_linear_amd import pipeline, tp
    torch.cuda.set_device(0)
    return tp, pipeline


def _qkv_bits(t):
    return np.ascontiguousarray(np.hstack([t["Wq"].data, t["Wk"].data, t["Wv"].data]))


def _qkv_values(t):
    return np.hstack([t["Wq"].values(), t["Wk"].values(), t["Wv"].values()])


def _sync():
    torch.cuda.synchronize()


# ============================================================== bit-exact indexing pins
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("world", [1, 2, 4])
def test_column_shard_onehot_exact(lib, dtype, world):
    """X = one-hot rows, so Y[t, j] = W[k(t), r N/P + j]: any misplaced shard, wrong offset,
    transposed slice or wrong leading dimension shows as a wrong value."""
    tp, pl = lib
    T, H, N = 300, 272, 784 if world != 4 else 800
    rng = np.random.Generator(np.random.PCG64(100 + world))
    X = np.zeros((T, H), np.float32)
    X[np.arange(T), (np.arange(T) * 37) % H] = 1.0
    Wv = from_values("W", rng.standard_normal((H, N)).astype(np.float32), dtype).values()
    Xd, Wd = dev_values(X, dtype), dev_values(Wv, dtype)
    Yfull = torch.full((T, N), -7.0, dtype=Xd.dtype, device=Xd.device)
    nl = N // world
    for r in range(world):
        say(f"  column one-hot dtype={dtype} world={world} rank={r} T={T} H={H} N={N}")
        tp.tp_col_linear_gelu(Xd, Wd, Yfull[:, r * nl:], N, T, H, N, r, world, tp.TP_ACT_NONE,
                              tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    ref = O.concat_columns([O.col_linear(X, Wv, r, world) for r in range(world)])
    check_exact(f"concat world={world}", Yfull, ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_column_writes_only_its_block(lib, dtype):
    """Only columns [0, N/P) of the rank's output view are written; the rest of Yfull keeps
    its sentinel."""
    tp, pl = lib
    T, H, N, P = 100, 64, 512, 4
    rng = np.random.Generator(np.random.PCG64(7))
    Xd = dev_values(rng.standard_normal((T, H)), dtype)
    Wd = dev_values(rng.standard_normal((H, N)), dtype)
    Y = torch.full((T, N), 3.0, dtype=Xd.dtype, device=Xd.device)
    say(f"  column writes only rank 2 block dtype={dtype}")
    tp.tp_col_linear_gelu(Xd, Wd, Y[:, 2 * 128:], N, T, H, N, 2, P, tp.TP_ACT_GELU_TANH,
                          tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    Yh = host(Y)
    assert np.all(Yh[:, :256] == 3.0) and np.all(Yh[:, 384:] == 3.0)
    assert not np.all(Yh[:, 256:384] == 3.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("world", [2, 4, 8])
def test_row_partials_integer_exact(lib, dtype, world):
    """Integer X in {-1,0,1} and W in {-2..2}: every partial and their sum are exact
    integers below 2^24, so the GPU must match the oracle bit for bit."""
    tp, pl = lib
    T, K, N = 260, 1088 if world != 8 else 1152, 392
    rng = np.random.Generator(np.random.PCG64(200 + world))
    X = integer_matrix(rng, (T, K), -1, 1, dtype)
    W = integer_matrix(rng, (K, N), -2, 2, dtype)
    Xd, Wd = dev(X), dev(W)
    sh = pl.LinearShard(Xd, Wd, world, dtype, col_ranks=())
    say(f"  row partials integer dtype={dtype} world={world} T={T} K={K} N={N}")
    sh.step()
    _sync()
    parts = [O.row_linear_partial(X.values(), W.values(), r, world) for r in range(world)]
    for r in range(world):
        check_exact(f"partial rank {r}", sh.parts[r], parts[r], "f32")
    check_exact("sum of partials", sh.Z, O.reduce_partials(parts), "f32")


@pytest.mark.parametrize("world", [2, 4])
def test_mlp_concat_integer_exact(lib, world):
    """Sparse integer X (8 nonzeros per row) and integer A: the column outputs are small
    integers, exact in bf16, so the concatenated hidden activation (no activation) is
    bit-exact; the row stage then reads exactly that buffer."""
    tp, pl = lib
    T, H, F = 300, 264, 1088
    rng = np.random.Generator(np.random.PCG64(300 + world))
    X = integer_matrix(rng, (T, H), -1, 1, "bf16", nnz_per_row=8)
    A = integer_matrix(rng, (H, F), -2, 2, "bf16")
    Xd, Ad = dev(X), dev(A)
    Yfull = torch.empty(T, F, dtype=torch.bfloat16, device="cuda:0")
    fl = F // world
    for r in range(world):
        say(f"  mlp concat integer world={world} rank={r}")
        tp.tp_col_linear_gelu(Xd, Ad, Yfull[:, r * fl:], F, T, H, F, r, world, tp.TP_ACT_NONE,
                              tp.TP_BF16)
    _sync()
    ref = O.concat_columns([O.col_linear(X.values(), A.values(), r, world) for r in range(world)])
    check_exact("hidden concat", Yfull, ref, "bf16")


# ============================================================== reduced-size workloads
def test_small_mlp_f32(lib):
    tp, pl = lib
    cfg = small_variant("mlp_f32_tp2")
    t = generate(cfg)
    sh = pl.MLPShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), cfg.world, "f32", residual_ln=False)
    say(f"  small fp32 MLP {cfg}")
    sh.step()
    _sync()
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    Y = O.concat_columns([O.col_linear(X, A, r, cfg.world, "gelu_tanh") for r in range(cfg.world)])
    check("hidden (GeLU)", sh.Yfull, Y, "f32")
    parts = [O.mlp_shard(X, A, B, r, cfg.world) for r in range(cfg.world)]
    for r in range(cfg.world):
        check(f"partial rank {r}", sh.parts[r], parts[r], "f32")
    check("Z", sh.Z, O.reduce_partials(parts), "f32")


def test_small_linear_bf16(lib):
    tp, pl = lib
    cfg = small_variant("linear_bf16_tp2")
    t = generate(cfg)
    sh = pl.LinearShard(dev(t["X"]), dev(t["W"]), cfg.world, "bf16", col_ranks=(0, 1))
    say(f"  small bf16 linear {cfg}")
    sh.step()
    _sync()
    X, W = t["X"].values(), t["W"].values()
    for r in (0, 1):
        check(f"column block rank {r}", sh.Ycol[r], O.col_linear(X, W, r, cfg.world), "bf16")
    parts = [O.row_linear_partial(X, W, r, cfg.world) for r in range(cfg.world)]
    for r in range(cfg.world):
        check(f"row partial rank {r}", sh.parts[r], parts[r], "bf16")
    check("Z", sh.Z, O.reduce_partials(parts), "bf16")


@pytest.mark.parametrize("affine", [False, True])
def test_small_mlp_bf16(lib, affine):
    tp, pl = lib
    cfg = small_variant("mlp_bf16_tp4")
    t = generate(cfg)
    if affine:
        t.update(random_affine(cfg, 5))
    sh = pl.MLPShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), cfg.world, "bf16",
                     gamma=dev(t["gamma"]), beta=dev(t["beta"]), eps=cfg.eps)
    say(f"  small bf16 MLP affine={affine} {cfg}")
    sh.step()
    _sync()
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    Y = O.concat_columns([O.col_linear(X, A, r, cfg.world, "gelu_tanh") for r in range(cfg.world)])
    check("hidden (GeLU)", sh.Yfull, Y, "bf16")
    parts = [O.mlp_shard(X, A, B, r, cfg.world) for r in range(cfg.world)]
    for r in range(cfg.world):
        check(f"partial rank {r}", sh.parts[r], parts[r], "bf16")
    h, y = O.reduce_residual_layernorm(parts, X, t["gamma"].values(), t["beta"].values(), cfg.eps)
    check("h = X + sum", sh.h, h, "bf16")
    check("y = LN(h)", sh.y, y, "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_small_attention(lib, causal):
    tp, pl = lib
    cfg = small_variant("attn_bf16_tp4").with_(causal=causal)
    t = generate(cfg)
    Xn = t["X"].values()
    Wqkv = _qkv_values(t)
    Wo = t["Wo"].values()
    sh = pl.AttnShard(dev(t["X"]), dev_values(Wqkv, "bf16"), dev(t["Wo"]), cfg.world, cfg.batch,
                      cfg.seq, cfg.n_heads, cfg.head_dim, causal)
    H, nb = cfg.hidden, (cfg.n_heads // cfg.world) * cfg.head_dim
    parts = []
    for r in range(cfg.world):
        say(f"  small attention causal={causal} rank={r} {cfg}")
        sh.rank(r)
        _sync()
        qkv, A = sh.workspace_views()
        h0 = r * nb
        ref_qkv = np.hstack([O.matmul(Xn, Wqkv[:, b * H + h0: b * H + h0 + nb]) for b in range(3)])
        check(f"QKV rank {r}", qkv, ref_qkv, "bf16")
        check(f"heads rank {r}", A, O.attention_heads(Xn, Wqkv, cfg.n_heads, cfg.head_dim, r,
                                                     cfg.world, cfg.batch, cfg.seq, causal), "bf16")
        parts.append(O.attn_head_shard(Xn, Wqkv, Wo, cfg.n_heads, cfg.head_dim, r, cfg.world,
                                       cfg.batch, cfg.seq, causal))
        check(f"O partial rank {r}", sh.parts[r], parts[r], "bf16")
    sh.reduce()
    _sync()
    check("sum of partials", sh.Z, O.reduce_partials(parts), "bf16")


def _block_runner(pl, cfg, t, sequence_parallel=False):
    return pl.BlockShard(dev(t["X"]), dev_values(_qkv_values(t), "bf16"), dev(t["Wo"]),
                         dev(t["W1"]), dev(t["W2"]), dev(t["gamma"]), dev(t["beta"]),
                         dev(t["gamma"]), dev(t["beta"]), cfg.world, cfg.batch, cfg.seq,
                         cfg.n_heads, cfg.head_dim, cfg.causal, cfg.eps,
                         sequence_parallel=sequence_parallel)


def _block_ref(cfg, t, rows=None):
    g, b = t["gamma"].values(), t["beta"].values()
    return O.block_shard(t["X"].values(), _qkv_values(t), t["Wo"].values(), t["W1"].values(),
                         t["W2"].values(), g, b, g, b, n_heads=cfg.n_heads,
                         head_dim=cfg.head_dim, world=cfg.world, batch=cfg.batch, seq=cfg.seq,
                         causal=cfg.causal, eps=cfg.eps, rows=rows)


def test_small_block(lib):
    tp, pl = lib
    cfg = small_variant("block_bf16_tp8")
    t = generate(cfg)
    sh = _block_runner(pl, cfg, t)
    ref = _block_ref(cfg, t)
    say(f"  small block: pre-LN + attention phase {cfg}")
    sh.attention_phase()
    _sync()
    check("xn = LN(X)", sh.xn, ref["xn"], "bf16")
    for r in range(cfg.world):
        check(f"attention partial rank {r}", sh.parts[r], ref["attn_parts"][r], "bf16")
    say("  small block: reduce1 + MLP phase + reduce2")
    sh.reduce1()
    sh.mlp_phase()
    _sync()
    check("h", sh.h, ref["h"], "bf16")
    check("hn", sh.hn, ref["hn"], "bf16")
    for r in range(cfg.world):
        check(f"MLP partial rank {r}", sh.parts[r], ref["mlp_parts"][r], "bf16")
    sh.reduce2()
    _sync()
    check("out", sh.out, ref["out"], "bf16")


def test_block_deterministic(lib):
    tp, pl = lib
    cfg = small_variant("block_bf16_tp8")
    t = generate(cfg)
    sh = _block_runner(pl, cfg, t)
    say("  block determinism: two steps")
    sh.step()
    _sync()
    first = sh.out.clone()
    sh.step()
    _sync()
    assert torch.equal(first.view(torch.int16), sh.out.view(torch.int16))


def test_block_sequence_parallel(lib):
    """The block with sequence-parallel epilogues (each rank reduce-scatters its rows; the
    row blocks land at their offsets, which is the all-gather) gives the same bits as the
    fused all-reduce epilogues, and matches the oracle's gathered reduce-scatter blocks."""
    tp, pl = lib
    cfg = small_variant("block_bf16_tp8")
    t = generate(cfg)
    full = _block_runner(pl, cfg, t)
    sp = _block_runner(pl, cfg, t, sequence_parallel=True)
    say(f"  block sequence-parallel vs all-reduce epilogues {cfg}")
    full.step()
    sp.step()
    _sync()
    for name in ("h", "hn", "out"):
        a, b = getattr(full, name), getattr(sp, name)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    ref = _block_ref(cfg, t)
    check("out (sequence parallel)", sp.out, ref["out"], "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,H,n_parts,world", [
    (64, 256, 4, 4),       # one row block per rank
    (96, 4104, 3, 8),      # 12 rows per rank, ragged vector tail
    (8192, 12288, 8, 8),   # the block's epilogue shape, 1024 rows per rank
])
def test_reduce_scatter_rows(lib, dtype, rows, H, n_parts, world):
    """Each rank's reduce-scatter + residual + LN gives exactly the rows the fused all-reduce
    epilogue gives for them, and the oracle's reduce-scatter blocks within tolerance."""
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(rows + H + world))
    Pd = (torch.randn(n_parts, rows, H, device="cuda:0") * 2).float()
    Rd = dev_values((rng.standard_normal((rows, H)) + 0.5).astype(np.float32), dtype)
    gd = dev_values((1 + 0.5 * rng.standard_normal(H)).astype(np.float32), dtype)
    bd = dev_values((0.5 * rng.standard_normal(H)).astype(np.float32), dtype)
    dt = tp.TP_BF16 if dtype == "bf16" else tp.TP_F32
    h_all = torch.empty(rows, H, dtype=Rd.dtype, device="cuda:0")
    y_all = torch.empty_like(h_all)
    tp.tp_partial_reduce_residual_ln(Pd, n_parts, rows * H, Rd, gd, bd, 1e-5, h_all, y_all, rows,
                                     H, dt)
    h_sp = torch.full_like(h_all, 7.0)
    y_sp = torch.full_like(h_all, 7.0)
    n = rows // world
    for r in range(world):
        say(f"  reduce-scatter dtype={dtype} rows={rows} H={H} parts={n_parts} rank={r}/{world}")
        tp.tp_partial_reduce_scatter_residual_ln(Pd, n_parts, rows * H, Rd, gd, bd, 1e-5,
                                                 h_sp[r * n:], y_sp[r * n:], rows, H, r, world, dt)
    _sync()
    assert torch.equal(h_all, h_sp) and torch.equal(y_all, y_sp)
    sample = [0, 1, world // 2, world - 1]
    parts_h = host(Pd) if rows * H <= 1 << 22 else None
    for r in sorted(set(sample)):
        rows_r = slice(r * n, (r + 1) * n)
        if parts_h is None:  # large case: the oracle on the first and last rows of the block
            idx = np.array([r * n, (r + 1) * n - 1])
            P = [host(Pd[p][idx]) for p in range(n_parts)]
            h, y = O.reduce_residual_layernorm(P, host(Rd[idx]), host(gd), host(bd), 1e-5)
            check(f"h rank {r} (rows)", h_sp[idx], h, dtype)
            check(f"y rank {r} (rows)", y_sp[idx], y, dtype)
            continue
        h, y = O.reduce_scatter_residual_layernorm(list(parts_h), host(Rd), host(gd), host(bd),
                                                   1e-5, r, world)
        check(f"h rank {r}", h_sp[rows_r], h, dtype)
        check(f"y rank {r}", y_sp[rows_r], y, dtype)


# ============================================================== edge cases
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,H,N,world,rank", [
    (1, 8, 8, 1, 0),          # smallest everything
    (1, 264, 16, 2, 1),       # single row, narrow shard
    (257, 64, 520, 1, 0),     # one row past a tile, world 1
    (33, 4104, 264, 3, 2),    # K past 64 ragged, odd world, last rank
    (513, 128, 4096, 8, 7),   # wide N, many ranks
])
def test_column_edge_shapes(lib, dtype, T, H, N, world, rank):
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(T * 7 + N))
    X = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((H, N)) / np.sqrt(H)).astype(np.float32)
    Xd, Wd = dev_values(X, dtype), dev_values(W, dtype)
    Xv, Wv = host(Xd), host(Wd)
    nl = N // world
    Y = torch.empty(T, nl + 8, dtype=Xd.dtype, device=Xd.device)  # ldy > width
    say(f"  column edge dtype={dtype} T={T} H={H} N={N} world={world} rank={rank}")
    tp.tp_col_linear_gelu(Xd, Wd, Y, nl + 8, T, H, N, rank, world, tp.TP_ACT_GELU_TANH,
                          tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    check("column", Y[:, :nl], O.col_linear(Xv, Wv, rank, world, "gelu_tanh"), dtype)


@pytest.mark.parametrize("T,N", [(448, 512), (512, 512), (64, 8), (1000, 40)])
def test_f32_small_and_tiled_kernels_integer_exact(lib, T, N):
    """The fp32 products take a 16 x 16-tile kernel with the contraction split over its waves
    when there are fewer 64 x 64 tiles than a quarter of the compute units (448 x 512: 56
    tiles), and the 64 x 64 tile otherwise (512 x 512: 64 tiles).  With integer operands every
    sum is exact in any order, so both must equal the oracle bit for bit: the column product
    with its GeLU off, and the row partial written and then accumulated onto itself (its
    fold epilogue).  K = 776 ends inside a 256-deep block of the split kernel."""
    tp, pl = lib
    K = 776
    rng = np.random.Generator(np.random.PCG64(3000 + T + N))
    X = integer_matrix(rng, (T, K), -1, 1, "f32")
    W = integer_matrix(rng, (K, 2 * N), -2, 2, "f32")
    Xd, Wd = dev(X), dev(W)
    Xv, Wv = X.values(), W.values()
    Y = torch.full((T, N), -5.0, dtype=torch.float32, device="cuda:0")
    say(f"  fp32 kernels T={T} K={K} N={N}: column rank 1 of 2")
    tp.tp_col_linear_gelu(Xd, Wd, Y, N, T, K, 2 * N, 1, 2, tp.TP_ACT_NONE, tp.TP_F32)
    _sync()
    check_exact("column rank 1", Y, O.col_linear(Xv, Wv, 1, 2), "f32")
    # row product: the full input [T, 2K] (rank 1's shard is its column block 1) against
    # W [2K, N]; the call reads the shard in place (leading dimension 2K)
    Xf = integer_matrix(rng, (T, 2 * K), -1, 1, "f32")
    Wr = integer_matrix(rng, (2 * K, N), -2, 2, "f32")
    Xfd, Wrd = dev(Xf), dev(Wr)
    Z = torch.empty(T, N, dtype=torch.float32, device="cuda:0")
    say(f"  fp32 kernels T={T} K={K} N={N}: row partial rank 1 of 2, then accumulated")
    tp.tp_row_linear_partial(Xfd[:, K:], 2 * K, Wrd, Z, T, 2 * K, N, 1, 2, tp.TP_F32)
    _sync()
    part = O.row_linear_partial(Xf.values(), Wr.values(), 1, 2)
    check_exact("row partial rank 1", Z, part, "f32")
    tp.tp_row_linear_fold(Xfd[:, K:], 2 * K, Wrd, Z, T, 2 * K, N, 1, 2, 1, tp.TP_F32)
    _sync()
    check_exact("row partial accumulated", Z, 2 * part, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N,world,rank", [
    (1, 8, 8, 1, 0),
    (5, 16, 24, 2, 1),
    (300, 1040, 136, 2, 0),   # K/world = 520: ragged K tile
    (64, 6144, 264, 8, 5),
])
def test_row_edge_shapes(lib, dtype, T, K, N, world, rank):
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(T * 11 + K))
    X = rng.standard_normal((T, K + 16)).astype(np.float32)  # ldx > K
    W = (rng.standard_normal((K, N)) / np.sqrt(K)).astype(np.float32)
    Xd, Wd = dev_values(X, dtype), dev_values(W, dtype)
    Xv, Wv = host(Xd), host(Wd)
    Z = torch.empty(T, N, dtype=torch.float32, device=Xd.device)
    say(f"  row edge dtype={dtype} T={T} K={K} N={N} world={world} rank={rank}")
    kl = K // world
    tp.tp_row_linear_partial(Xd[:, rank * kl:], K + 16, Wd, Z, T, K, N, rank, world,
                             tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    check("row partial", Z, O.row_linear_partial(Xv[:, :K], Wv, rank, world), dtype)


def test_f32_column_many_row_tiles(lib):
    """An fp32 column call with more row tiles (65600 of 64 rows) than one grid dimension
    holds: every tile is computed (sampled rows, including the last tile, against the
    oracle)."""
    tp, pl = lib
    T, H, N = 64 * 65600 - 24, 8, 16
    rng = np.random.Generator(np.random.PCG64(65600))
    X = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((H, N)) / np.sqrt(H)).astype(np.float32)
    Xd, Wd = dev_values(X, "f32"), dev_values(W, "f32")
    Y = torch.full((T, N // 2), float("nan"), dtype=torch.float32, device=Xd.device)
    say(f"  fp32 column with many row tiles T={T} H={H} N={N}")
    tp.tp_col_linear_gelu(Xd, Wd, Y, N // 2, T, H, N, 1, 2, tp.TP_ACT_GELU_TANH, tp.TP_F32)
    _sync()
    assert bool(torch.isfinite(Y).all())
    rows = np.unique(np.concatenate([np.arange(0, T, 4093), np.arange(T - 70, T)]))
    check("column (rows)", Y[rows], O.col_linear(X.astype(np.float64), W.astype(np.float64),
                                                 1, 2, "gelu_tanh", rows), "f32")


@pytest.mark.parametrize("T,H,nl,tile", [
    (8190, 136, 1016, "256x128"),  # 32 x 8 tiles of 256 x 128, ragged rows and columns
    (8190, 136, 1528, "256x192"),  # 32 x 8 tiles of 256 x 192
    (8190, 136, 2040, "256x256"),  # 32 x 8 tiles of 256 x 256
])
@pytest.mark.parametrize("mode", ["none", "gelu", "save"])
def test_column_tile_widths(lib, T, H, nl, tile, mode):
    """Every bf16 column epilogue (plain, GeLU, GeLU keeping the pre-activation) at each tile
    width the launch planner picks on 256 compute units, with ragged last rows, columns and
    K, rank 1 of 2 and a leading dimension past the shard width.  The 256 x 128 and 256 x 256
    tiles write their outputs through LDS, the 256 x 192 tile directly."""
    tp, pl = lib
    world, rank = 2, 1
    N = world * nl
    rng = np.random.Generator(np.random.PCG64(T + nl))
    X = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((H, N)) / np.sqrt(H)).astype(np.float32)
    Xd, Wd = dev_values(X, "bf16"), dev_values(W, "bf16")
    Xv, Wv = host(Xd), host(Wd)
    ld = nl + 8
    Y = torch.full((T, ld), float("nan"), dtype=torch.bfloat16, device=Xd.device)
    U = torch.full((T, ld), float("nan"), dtype=torch.bfloat16, device=Xd.device)
    say(f"  column tile widths T={T} H={H} N/P={nl} ({tile} tiles) mode={mode}")
    if mode == "save":
        tp.tp_col_linear_gelu_save(Xd, Wd, Y, ld, U, ld, T, H, N, rank, world, tp.TP_BF16)
    else:
        act = tp.TP_ACT_GELU_TANH if mode == "gelu" else tp.TP_ACT_NONE
        tp.tp_col_linear_gelu(Xd, Wd, Y, ld, T, H, N, rank, world, act, tp.TP_BF16)
    _sync()
    act = "none" if mode == "none" else "gelu_tanh"
    check("column", Y[:, :nl], O.col_linear(Xv, Wv, rank, world, act), "bf16")
    assert torch.isnan(Y[:, nl:].float()).all(), "column wrote past its shard width"
    if mode == "save":
        check("pre-activation", U[:, :nl], O.col_linear(Xv, Wv, rank, world), "bf16")
        assert torch.isnan(U[:, nl:].float()).all(), "pre-activation written past its width"


def test_column_split_launch(lib):
    """A product whose columns the launcher splits over two launches: 4096 columns of
    256 x 256 tiles (one full round on 256 compute units) and a 512-wide strip of 128 x 128
    tiles.  (The full-size attention and block tests take the same split through the QKV
    column-block map.)"""
    tp, pl = lib
    T, H, nh, d, world, rank = 4096, 256, 24, 128, 2, 1  # H_model = nh*d = 3072; rank block 1536
    Hm = nh * d
    rng = np.random.Generator(np.random.PCG64(4608))
    X = rng.standard_normal((T, Hm)).astype(np.float32)
    Wqkv = (rng.standard_normal((Hm, 3 * Hm)) / np.sqrt(Hm)).astype(np.float32)
    Xd, Wd = dev_values(X, "bf16"), dev_values(Wqkv, "bf16")
    Xv, Wv = host(Xd), host(Wd)
    nl = 3 * Hm // world  # 4608 output columns
    Y = torch.empty(T, nl, dtype=torch.bfloat16, device=Xd.device)
    say(f"  column split launch T={T} H={Hm} N/P={nl}")
    tp.tp_col_linear_gelu(Xd, Wd, Y, nl, T, Hm, 3 * Hm, rank, world, tp.TP_ACT_GELU_TANH, tp.TP_BF16)
    _sync()
    check("column (split launch)", Y, O.col_linear(Xv, Wv, rank, world, "gelu_tanh"), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N,world,rank", [(70, 1024, 264, 4, 3), (300, 6144, 136, 8, 2)])
def test_row_dense_shard(lib, dtype, T, K, N, world, rank):
    """The rank's input shard held as its own dense [T, K/world] buffer (ldx = K/world), as
    the block keeps each rank's hidden activation."""
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(T * 7 + K + rank))
    kl = K // world
    X = rng.standard_normal((T, K)).astype(np.float32)
    W = (rng.standard_normal((K, N)) / np.sqrt(K)).astype(np.float32)
    Xd, Wd = dev_values(X, dtype), dev_values(W, dtype)
    Xv, Wv = host(Xd), host(Wd)
    Xr = Xd[:, rank * kl:(rank + 1) * kl].contiguous()
    Z = torch.empty(T, N, dtype=torch.float32, device=Xd.device)
    say(f"  row dense shard dtype={dtype} T={T} K={K} N={N} world={world} rank={rank}")
    tp.tp_row_linear_partial(Xr, kl, Wd, Z, T, K, N, rank, world,
                             tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    check("row partial (dense shard)", Z, O.row_linear_partial(Xv, Wv, rank, world), dtype)


@pytest.mark.parametrize("seq", [2048, 2000])  # whole 256-row tiles; a ragged last tile
def test_attention_qkv_split_strip(lib, seq):
    """The attention shard's QKV projection when its launch plan has a narrow strip (on 256
    compute units: 8192 columns of 256 x 256 tiles plus a 256-wide strip): the strip's
    contraction is split over 4 ranges into fp32 partials in the workspace and summed into
    the bf16 QKV by the reduce kernel.  The QKV in the workspace and the output partial are
    checked on sampled rows against the oracle."""
    tp, pl = lib
    batch, nh, d, world, rank = 1, 22, 128, 1, 0
    H = nh * d  # 2816: the rank's QKV is 2048 x 8448, contraction 2816
    T = batch * seq
    rng = np.random.Generator(np.random.PCG64(2816 + seq))
    X = rng.standard_normal((T, H)).astype(np.float32)
    Wqkv = (rng.standard_normal((H, 3 * H)) / np.sqrt(H)).astype(np.float32)
    Wo = (rng.standard_normal((H, H)) / np.sqrt(H)).astype(np.float32)
    Xd, Wqd, Wod = dev_values(X, "bf16"), dev_values(Wqkv, "bf16"), dev_values(Wo, "bf16")
    Xv, Wqv, Wov = host(Xd), host(Wqd), host(Wod)
    plain = (T * 3 * H * 2 + T * H * 2 + 255) // 256 * 256
    ws_bytes = tp.tp_attn_workspace_bytes(batch, seq, H, nh, d, world, tp.TP_BF16)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert ws_bytes == plain + 4 * T * 256 * 4, "workspace has no room for the split strip"
    sh = pl.AttnShard(Xd, Wqd, Wod, world, batch, seq, nh, d, True)
    say(f"  attention QKV with a split strip T={T} H={H} heads={nh}")
    sh.step()
    _sync()
    rows = sample_rows(T, seq, 5)
    QKV, _ = sh.workspace_views()
    lo, hi = O.head_range(nh, world, rank)
    Wr = np.hstack([blk[:, lo * d:hi * d] for blk in O.split_qkv(Wqv, H)])
    check("QKV (rows)", QKV[rows], O.matmul(Xv[rows], Wr), "bf16")
    check("partial (rows)", sh.parts[rank][rows],
          O.attn_head_shard(Xv, Wqv, Wov, nh, d, rank, world, batch, seq, True, rows), "bf16")


def test_attention_qkv_split_strip_integer_exact(lib):
    """Integer pin of the split strip: with X sparse in {-1, 0, 1} (8 nonzeros per row) and
    Wqkv in {-2..2}, every partial of every contraction range and their sum are small
    integers, exact in fp32 and in bf16, so the whole QKV of rank 1 of 2 (its head blocks of
    [Wq | Wk | Wv] through the column-block map, strip included) equals the oracle bit for bit.
    A wrong contraction range, split offset or partial slot shows up as a wrong integer."""
    tp, pl = lib
    batch, seq, nh, d, world, rank = 1, 2048, 44, 128, 2, 1
    H = nh * d  # 5632; the rank's QKV is 2048 x 8448 (8192 columns + a 256-wide strip)
    T = batch * seq
    rng = np.random.Generator(np.random.PCG64(44))
    X = integer_matrix(rng, (T, H), -1, 1, "bf16", nnz_per_row=8)
    Wqkv = integer_matrix(rng, (H, 3 * H), -2, 2, "bf16")
    Wo = integer_matrix(rng, (H, H), -1, 1, "bf16")
    sh = pl.AttnShard(dev(X), dev(Wqkv), dev(Wo), world, batch, seq, nh, d, True)
    say(f"  attention QKV split strip, integer inputs T={T} H={H} rank {rank}/{world}")
    sh.rank(rank)
    _sync()
    QKV, _ = sh.workspace_views()
    lo, hi = O.head_range(nh, world, rank)
    Wr = np.hstack([blk[:, lo * d:hi * d] for blk in O.split_qkv(Wqkv.values(), H)])
    check_exact("QKV (integer)", QKV, O.matmul(X.values(), Wr), "bf16")


@pytest.mark.parametrize("batch,seq,n_heads,world,causal", [
    (1, 1, 2, 1, True),        # one token
    (3, 65, 4, 2, True),       # one key past a key block, three sequences
    (2, 130, 2, 2, False),     # one query past a query block, full attention
    (1, 257, 8, 8, True),      # one head per rank
    (2, 300, 16, 2, True),     # 16 (sequence, head) pairs, ragged last block
    (4, 129, 8, 4, False),     # 8 pairs, full attention, one query past a block
])
def test_attention_edge_shapes(lib, batch, seq, n_heads, world, causal):
    tp, pl = lib
    d = 128
    H = n_heads * d
    rng = np.random.Generator(np.random.PCG64(seq * 13 + n_heads))
    Xn = rng.standard_normal((batch * seq, H)).astype(np.float32)
    Wqkv = (rng.standard_normal((H, 3 * H)) / np.sqrt(H)).astype(np.float32)
    Wo = (rng.standard_normal((H, H)) / np.sqrt(H)).astype(np.float32)
    Xd, Wqd, Wod = dev_values(Xn, "bf16"), dev_values(Wqkv, "bf16"), dev_values(Wo, "bf16")
    Xv, Wqv, Wov = host(Xd), host(Wqd), host(Wod)
    sh = pl.AttnShard(Xd, Wqd, Wod, world, batch, seq, n_heads, d, causal)
    for r in range(world):
        say(f"  attention edge batch={batch} seq={seq} heads={n_heads} world={world} rank={r} causal={causal}")
        sh.rank(r)
        _sync()
        _, A = sh.workspace_views()
        check(f"heads rank {r}", A, O.attention_heads(Xv, Wqv, n_heads, d, r, world, batch, seq,
                                                     causal), "bf16")
        check(f"partial rank {r}", sh.parts[r], O.attn_head_shard(Xv, Wqv, Wov, n_heads, d, r,
                                                                  world, batch, seq, causal), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,H,n_parts,residual,ln", [
    (5, 8, 0, True, True),        # plain LayerNorm of a narrow row
    (20000, 64, 0, True, True),   # LayerNorm, several rows per workgroup (odd and even counts)
    (1000, 12288, 0, True, True), # LayerNorm at the block's width, more rows than resident groups
    (777, 4104, 0, True, False),  # no partials, no LayerNorm: h = residual, ragged vector tail
    (300, 12288, 1, True, True),  # one partial, wide row
    (64, 4104, 3, False, True),   # no residual, ragged vector tail
    (17, 65536, 2, True, True),   # widest supported row (1024-thread path)
    (100, 256, 8, True, False),   # sum only, h_out
])
def test_reduce_edge_cases(lib, dtype, rows, H, n_parts, residual, ln):
    tp, pl = lib
    rng = np.random.Generator(np.random.PCG64(rows * 3 + H + n_parts))
    parts = (rng.standard_normal((max(n_parts, 1), rows, H)) * 2).astype(np.float32)
    R = (rng.standard_normal((rows, H)) + 0.5).astype(np.float32)
    g = (1 + 0.5 * rng.standard_normal(H)).astype(np.float32)
    b = (0.5 * rng.standard_normal(H)).astype(np.float32)
    Pd = torch.from_numpy(parts).to("cuda:0")
    Rd, gd, bd = dev_values(R, dtype), dev_values(g, dtype), dev_values(b, dtype)
    hd = torch.empty(rows, H, dtype=Rd.dtype, device="cuda:0")
    yd = torch.empty_like(hd)
    say(f"  reduce edge dtype={dtype} rows={rows} H={H} parts={n_parts} residual={residual} ln={ln}")
    tp.tp_partial_reduce_residual_ln(Pd if n_parts else None, n_parts, rows * H,
                                     Rd if residual else None, gd if ln else None,
                                     bd if ln else None, 1e-5, hd, yd if ln else None, rows, H,
                                     tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    h, y = O.reduce_residual_layernorm(list(parts[:n_parts]), host(Rd) if residual else None,
                                       host(gd) if ln else None, host(bd) if ln else None, 1e-5)
    check("h", hd, h, dtype)
    if ln:
        check("y", yd, y, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H", [512, 1024, 2048, 4096, 6144, 8192, 12288, 16384, 24576, 32768])
def test_reduce_every_full_width(lib, dtype, H):
    """Rows that every thread's runs fill exactly, for each launch shape (64 to 1024 threads, 1
    to 8 runs): over fp32 partials a run is two 4-element halves 256 apart, which every output
    element must see the same as a ragged row would."""
    tp, pl = lib
    rows, n_parts = 37, 3
    rng = np.random.Generator(np.random.PCG64(4100 + H))
    parts = (rng.standard_normal((n_parts, rows, H)) * 2).astype(np.float32)
    R = (rng.standard_normal((rows, H)) + 0.5).astype(np.float32)
    g = (1 + 0.5 * rng.standard_normal(H)).astype(np.float32)
    b = (0.5 * rng.standard_normal(H)).astype(np.float32)
    Pd = torch.from_numpy(parts).to("cuda:0")
    Rd, gd, bd = dev_values(R, dtype), dev_values(g, dtype), dev_values(b, dtype)
    hd = torch.empty(rows, H, dtype=Rd.dtype, device="cuda:0")
    yd = torch.empty_like(hd)
    say(f"  reduce full width dtype={dtype} rows={rows} H={H} parts={n_parts}")
    tp.tp_partial_reduce_residual_ln(Pd, n_parts, rows * H, Rd, gd, bd, 1e-5, hd, yd, rows, H,
                                     tp.TP_BF16 if dtype == "bf16" else tp.TP_F32)
    _sync()
    h, y = O.reduce_residual_layernorm(list(parts), host(Rd), host(gd), host(bd), 1e-5)
    check("h", hd, h, dtype)
    check("y", yd, y, dtype)


@pytest.mark.parametrize("H", [4096, 12288])
def test_reduce_layouts_agree(lib, H):
    """The same bf16-valued partials reduced as fp32 partials (two-half runs) and as bf16
    partials (8 consecutive elements per run): each element's additions are the same, so h is
    bit-identical; the LayerNorm statistics are summed in another lane order, so y may differ
    by one bf16 step."""
    tp, pl = lib
    rows, n_parts = 129, 8
    rng = np.random.Generator(np.random.PCG64(4200 + H))
    P16 = dev_values(rng.standard_normal((n_parts, rows, H)), "bf16")
    P32 = P16.float()
    Rd = dev_values(rng.standard_normal((rows, H)), "bf16")
    gd = dev_values(1 + 0.5 * rng.standard_normal(H), "bf16")
    bd = dev_values(0.5 * rng.standard_normal(H), "bf16")
    h32, y32, h16, y16 = (torch.empty(rows, H, dtype=torch.bfloat16, device="cuda:0")
                          for _ in range(4))
    say(f"  reduce layouts fp32 / bf16 partials rows={rows} H={H}")
    tp.tp_partial_reduce_residual_ln(P32, n_parts, rows * H, Rd, gd, bd, 1e-5, h32, y32, rows, H,
                                     tp.TP_BF16)
    tp.tp_partial_reduce_residual_ln_bf16(P16, n_parts, rows * H, Rd, gd, bd, 1e-5, h16, y16,
                                          rows, H)
    _sync()
    assert torch.equal(h32.view(torch.int16), h16.view(torch.int16)), "h differs"
    # one bf16 step of |y| is at most 2^-7 |y|; near zero the fp32 statistics' own rounding
    # (about 1e-6 of the row's scale) decides instead
    a, b = y32.float(), y16.float()
    excess = ((a - b).abs() - (2.0 ** -7 * torch.maximum(a.abs(), b.abs()) + 1e-5)).max()
    assert float(excess) <= 0, f"y differs by more than one bf16 step ({float(excess)})"


def test_errors_leave_outputs_untouched(lib):
    tp, pl = lib
    Xd = torch.ones(64, 256, dtype=torch.bfloat16, device="cuda:0")
    Wd = torch.ones(256, 1024, dtype=torch.bfloat16, device="cuda:0")
    Y = torch.full((64, 512), 5.0, dtype=torch.bfloat16, device="cuda:0")
    say("  invalid calls on real buffers")
    with pytest.raises(tp.TPError):
        tp.tp_col_linear_gelu(Xd, Wd, Y, 512, 64, 256, 1024, 2, 2, 0, tp.TP_BF16)
    with pytest.raises(tp.TPError):
        tp.tp_col_linear_gelu(Xd, Wd, Y, 500, 64, 256, 1000, 0, 2, 0, tp.TP_BF16)
    _sync()
    assert torch.all(Y == 5.0)


# ============================================================== full-size workloads
FULL = pytest.mark.timeout(600)


@FULL
def test_full_mlp_f32(lib):
    tp, pl = lib
    cfg = get_config("mlp_f32_tp2")
    t = generate(cfg)
    sh = pl.MLPShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), cfg.world, "f32", residual_ln=False)
    say(f"  full fp32 MLP {cfg.name}")
    sh.step()
    _sync()
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    Y = O.concat_columns([O.col_linear(X, A, r, cfg.world, "gelu_tanh") for r in range(cfg.world)])
    check("hidden (GeLU)", sh.Yfull, Y, "f32")
    parts = [O.mlp_shard(X, A, B, r, cfg.world) for r in range(cfg.world)]
    for r in range(cfg.world):
        check(f"partial rank {r}", sh.parts[r], parts[r], "f32")
    check("Z", sh.Z, O.reduce_partials(parts), "f32")


@FULL
def test_full_linear_bf16(lib):
    tp, pl = lib
    cfg = get_config("linear_bf16_tp2")
    t = generate(cfg)
    sh = pl.LinearShard(dev(t["X"]), dev(t["W"]), cfg.world, "bf16", col_ranks=(0,))
    say(f"  full bf16 linear {cfg.name}")
    sh.step()
    _sync()
    # every element: 0.2 TFLOP of float64 oracle
    X, W = t["X"].values(), t["W"].values()
    check("column rank 0", sh.Ycol[0], O.col_linear(X, W, 0, 2), "bf16")
    parts = [O.row_linear_partial(X, W, r, 2) for r in range(2)]
    for r in range(2):
        check(f"row partial {r}", sh.parts[r], parts[r], "bf16")
    check("Z", sh.Z, O.reduce_partials(parts), "bf16")


@FULL
def test_full_mlp_bf16(lib):
    tp, pl = lib
    cfg = get_config("mlp_bf16_tp4")
    t = generate(cfg)
    sh = pl.MLPShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), cfg.world, "bf16",
                     gamma=dev(t["gamma"]), beta=dev(t["beta"]), eps=cfg.eps)
    say(f"  full bf16 MLP {cfg.name}")
    sh.step()
    _sync()
    # every element: 1.1 TFLOP of float64 oracle for the 4 ranks
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    Y = O.concat_columns([O.col_linear(X, A, r, cfg.world, "gelu_tanh")
                          for r in range(cfg.world)])
    check("hidden", sh.Yfull, Y, "bf16")
    parts = [O.row_linear_partial(Y, B, r, cfg.world) for r in range(cfg.world)]
    del Y
    for r in range(cfg.world):
        check(f"partial rank {r}", sh.parts[r], parts[r], "bf16")
    h, y = O.reduce_residual_layernorm(parts, X, t["gamma"].values(), t["beta"].values(),
                                       cfg.eps)
    check("h", sh.h, h, "bf16")
    check("y", sh.y, y, "bf16")


@FULL
def test_full_attention(lib):
    tp, pl = lib
    cfg = get_config("attn_bf16_tp4")
    t = generate(cfg)
    Xn, Wqkv, Wo = t["X"].values(), _qkv_values(t), t["Wo"].values()
    sh = pl.AttnShard(dev(t["X"]), dev_values(Wqkv, "bf16"), dev(t["Wo"]), cfg.world, cfg.batch,
                      cfg.seq, cfg.n_heads, cfg.head_dim, cfg.causal)
    say(f"  full attention {cfg.name}")
    sh.step()
    _sync()
    # every element: 2.2 TFLOP of float64 oracle for the 4 ranks
    _, A = sh.workspace_views()
    r_last = cfg.world - 1
    check(f"heads rank {r_last}", A,
          O.attention_heads(Xn, Wqkv, cfg.n_heads, cfg.head_dim, r_last, cfg.world, cfg.batch,
                            cfg.seq, True), "bf16")
    parts = []
    for r in range(cfg.world):
        parts.append(O.attn_head_shard(Xn, Wqkv, Wo, cfg.n_heads, cfg.head_dim, r, cfg.world,
                                       cfg.batch, cfg.seq, True))
        check(f"partial rank {r}", sh.parts[r], parts[r], "bf16")
    check("sum", sh.Z, O.reduce_partials(parts), "bf16")


@FULL
def test_full_block(lib):
    tp, pl = lib
    cfg = get_config("block_bf16_tp8")
    t = generate(cfg)
    say(f"  full block {cfg.name}: inputs generated")
    sh = _block_runner(pl, cfg, t)
    sh.attention_phase()
    _sync()
    # every element of every stage: 30 TFLOP of float64 oracle for the 8 ranks, computed
    # while the attention partials are still in their buffers (the MLP phase reuses them)
    say("  full block: attention phase done, computing the oracle's block")
    ref = _block_ref(cfg, t)
    check("xn", sh.xn, ref["xn"], "bf16")
    for r in range(cfg.world):
        check(f"attention partial {r}", sh.parts[r], ref["attn_parts"][r], "bf16")
    say("  full block: running reduce + MLP")
    sh.reduce1()
    sh.mlp_phase()
    sh.reduce2()
    _sync()
    check("h", sh.h, ref["h"], "bf16")
    check("hn", sh.hn, ref["hn"], "bf16")
    for r in range(cfg.world):
        check(f"MLP partial {r}", sh.parts[r], ref["mlp_parts"][r], "bf16")
    check("out", sh.out, ref["out"], "bf16")
