"""GPU parity of the backward pass of the column/row pair (the HIP library through its C ABI
against the float64 CPU oracle's chain-rule definitions).

  * integer inputs make every product exact: the input-gradient (dZ . W^T, dU . W^T) and
    weight-gradient (Y^T . dZ, X^T . dU) products must match bit for bit, which pins the
    transposed-operand layouts, the rank blocks and the ragged tails;
  * random inputs with the GeLU derivative fused: the tolerance rule of gpu_helpers.check;
  * the whole MLP (forward keeping the pre-activation, backward of every rank, reduce of the
    input-gradient partials) against the oracle's mlp_backward;
  * the full-size block MLP shard (T 8192, H 12288, F 49152, 8 ranks) on every element,
    launched as the bench launches it.
Inputs of the oracle are always the seeded synthetic tensors, never a GPU result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
from gpu_helpers import check, check_exact, dev, dev_values, host, say
from workloads import generate, get_config, output_gradient
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


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ============================================================== bit-exact layouts
@pytest.mark.parametrize("seq,K,N,world", [(300, 1088, 392, 4), (64, 512, 136, 2),
                                           (520, 2304, 264, 8)])
def test_row_backward_integer_exact(lib, seq, K, N, world):
    """Sparse integer dZ (8 nonzeros per row) and integer W, Y: dY = dZ . W_r^T is a small
    integer (exact in bf16) and dW_r = Y_r^T . dZ an integer below 2^24 (exact in fp32)."""
    tp, pl = lib
    rng = _rng(500 + world)
    dZ = integer_matrix(rng, (seq, N), -2, 2, "bf16", nnz_per_row=8)
    W = integer_matrix(rng, (K, N), -2, 2, "bf16")
    kl = K // world
    dZd, Wd = dev(dZ), dev(W)
    for r in range(world):
        Y = integer_matrix(rng, (seq, kl), -1, 1, "bf16")
        Yd = dev(Y)
        dY = torch.full((seq, kl), 5.0, dtype=torch.bfloat16, device="cuda:0")
        dW = torch.full((kl, N), 5.0, dtype=torch.float32, device="cuda:0")
        say(f"  row backward integer seq={seq} K={K} N={N} world={world} rank={r}")
        tp.tp_row_linear_backward(dZd, Wd, Yd, kl, None, 0, dY, kl, dW, N, seq, K, N, r, world,
                                  tp.TP_ACT_NONE, 0, tp.TP_BF16)
        _sync()
        rdY, rdW = O.row_linear_backward(dZ.values(), Y.values(), W.values(), r, world)
        check_exact(f"dY rank {r}", dY, rdY, "bf16")
        check_exact(f"dW rank {r}", dW, rdW, "f32")


@pytest.mark.parametrize("seq,H,N,world", [(300, 264, 1088, 4), (72, 136, 528, 2),
                                           (264, 520, 2048, 8)])
def test_col_backward_integer_exact(lib, seq, H, N, world):
    """Integer X, W and sparse integer dU: dX_part = dU . W_r^T and dW_r = X^T . dU are
    integers below 2^24, exact in fp32; the partials summed over ranks give dU . W^T."""
    tp, pl = lib
    rng = _rng(600 + world)
    X = integer_matrix(rng, (seq, H), -2, 2, "bf16")
    W = integer_matrix(rng, (H, N), -2, 2, "bf16")
    nl = N // world
    Xd, Wd = dev(X), dev(W)
    dU_full = integer_matrix(rng, (seq, N), -2, 2, "bf16", nnz_per_row=16)
    dUd = dev(dU_full)
    parts = torch.full((world, seq, H), 9.0, dtype=torch.float32, device="cuda:0")
    dWfull = torch.full((H, N), 9.0, dtype=torch.float32, device="cuda:0")
    for r in range(world):
        say(f"  col backward integer seq={seq} H={H} N={N} world={world} rank={r}")
        tp.tp_col_linear_backward(Xd, Wd, dUd[:, r * nl:], N, parts[r], dWfull[:, r * nl:], N,
                                  seq, H, N, r, world, 0, tp.TP_BF16)
    _sync()
    ref_parts = []
    for r in range(world):
        rdX, rdW = O.col_linear_backward(dU_full.values()[:, r * nl:(r + 1) * nl], X.values(),
                                         W.values(), r, world)
        check_exact(f"dX part rank {r}", parts[r], rdX, "f32")
        ref_parts.append(rdX)
        check_exact(f"dW block rank {r}", dWfull[:, r * nl:(r + 1) * nl], rdW, "f32")
    dX = torch.empty(seq, H, dtype=torch.float32, device="cuda:0")
    tp.tp_partial_reduce_residual_ln(parts, world, seq * H, None, None, None, 0.0, dX, None, seq,
                                     H, tp.TP_F32)
    _sync()
    check_exact("dX (sum of partials)", dX, O.reduce_partials(ref_parts), "f32")


# ============================================================== random inputs, GeLU fused
@pytest.mark.parametrize("seq,K,N,world,rank", [(300, 1088, 264, 4, 1), (200, 2048, 520, 8, 7),
                                                (40, 256, 72, 1, 0)])
def test_row_backward_gelu(lib, seq, K, N, world, rank):
    tp, pl = lib
    rng = _rng(700 + rank)
    kl = K // world
    dZ = rng.standard_normal((seq, N))
    W = rng.standard_normal((K, N)) / np.sqrt(N)
    U = 1.5 * rng.standard_normal((seq, kl))
    Y = rng.standard_normal((seq, kl))
    dZd, Wd, Ud, Yd = (dev_values(v, "bf16") for v in (dZ, W, U, Y))
    dZv, Wv, Uv, Yv = (host(t) for t in (dZd, Wd, Ud, Yd))  # the bf16 values both sides use
    dY = torch.empty(seq, kl, dtype=torch.bfloat16, device="cuda:0")
    dW = torch.empty(kl, N, dtype=torch.float32, device="cuda:0")
    say(f"  row backward gelu seq={seq} K={K} N={N} world={world} rank={rank}")
    tp.tp_row_linear_backward(dZd, Wd, Yd, kl, Ud, kl, dY, kl, dW, N, seq, K, N, rank, world,
                              tp.TP_ACT_GELU_TANH, 0, tp.TP_BF16)
    _sync()
    rdY, rdW = O.row_linear_backward(dZv, Yv, Wv, rank, world, Uv, "gelu_tanh")
    check("dY (GeLU' fused)", dY, rdY, "bf16")
    check("dW", dW, rdW, "f32")


def test_row_backward_single_outputs_and_accumulate(lib):
    """dY alone, dW alone, and dW accumulated onto an existing gradient (dW0 + Y^T dZ),
    written only inside the rank's block of a wider buffer."""
    tp, pl = lib
    seq, K, N, world, rank = 136, 1024, 200, 4, 2
    rng = _rng(710)
    kl = K // world
    dZ, W, Y = rng.standard_normal((seq, N)), rng.standard_normal((K, N)), rng.standard_normal((seq, kl))
    dZd, Wd, Yd = (dev_values(v, "bf16") for v in (dZ, W, Y))
    dZv, Wv, Yv = (host(t) for t in (dZd, Wd, Yd))
    rdY, rdW = O.row_linear_backward(dZv, Yv, Wv, rank, world)
    dY = torch.empty(seq, kl, dtype=torch.bfloat16, device="cuda:0")
    say("  row backward dY only")
    tp.tp_row_linear_backward(dZd, Wd, None, 0, None, 0, dY, kl, None, 0, seq, K, N, rank, world,
                              tp.TP_ACT_NONE, 0, tp.TP_BF16)
    ld = N + 24
    dW0 = rng.standard_normal((kl, ld)).astype(np.float32)
    dW = torch.from_numpy(dW0).to("cuda:0")
    say("  row backward dW only, accumulated")
    tp.tp_row_linear_backward(dZd, Wd, Yd, kl, None, 0, None, 0, dW, ld, seq, K, N, rank, world,
                              tp.TP_ACT_NONE, 1, tp.TP_BF16)
    _sync()
    check("dY only", dY, rdY, "bf16")
    got = host(dW)
    check("dW accumulated", got[:, :N], dW0[:, :N].astype(np.float64) + rdW, "f32")
    assert np.array_equal(got[:, N:], dW0[:, N:].astype(np.float64)), "wrote outside its block"


def test_col_backward_accumulate_twice(lib):
    """Two accumulating calls give dW0 + 2 X^T dU."""
    tp, pl = lib
    seq, H, N, world, rank = 264, 392, 1024, 4, 3
    rng = _rng(720)
    nl = N // world
    X, W, dU = rng.standard_normal((seq, H)), rng.standard_normal((H, N)), rng.standard_normal((seq, nl))
    Xd, Wd, dUd = (dev_values(v, "bf16") for v in (X, W, dU))
    Xv, Wv, dUv = (host(t) for t in (Xd, Wd, dUd))
    dW0 = rng.standard_normal((H, nl)).astype(np.float32)
    dW = torch.from_numpy(dW0).to("cuda:0")
    dXp = torch.empty(seq, H, dtype=torch.float32, device="cuda:0")
    for i in range(2):
        say(f"  col backward accumulate call {i + 1}")
        tp.tp_col_linear_backward(Xd, Wd, dUd, nl, dXp if i == 0 else None, dW, nl, seq, H, N,
                                  rank, world, 1, tp.TP_BF16)
    _sync()
    rdX, rdW = O.col_linear_backward(dUv, Xv, Wv, rank, world)
    check("dX part", dXp, rdX, "f32")
    check("dW0 + 2 X^T dU", dW, dW0.astype(np.float64) + 2 * rdW, "f32")


@pytest.mark.parametrize("world", [2, 4])
def test_col_gelu_save(lib, world):
    """The saving forward writes the same Y as tp_col_linear_gelu (bit for bit) and the
    pre-activation U = X . W_r."""
    tp, pl = lib
    cfg = small_variant("mlp_bf16_tp4")
    t = generate(cfg)
    T, H, F = cfg.tokens, cfg.hidden, cfg.ffn
    fl = F // world
    Xd, Ad = dev(t["X"]), dev(t["A"])
    for r in range(world):
        Y1 = torch.empty(T, fl, dtype=torch.bfloat16, device="cuda:0")
        Y2, U = torch.empty_like(Y1), torch.empty_like(Y1)
        say(f"  column GeLU with saved pre-activation world={world} rank={r}")
        tp.tp_col_linear_gelu(Xd, Ad, Y1, fl, T, H, F, r, world, tp.TP_ACT_GELU_TANH, tp.TP_BF16)
        tp.tp_col_linear_gelu_save(Xd, Ad, Y2, fl, U, fl, T, H, F, r, world, tp.TP_BF16)
        _sync()
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16)), "Y differs"
        check(f"U rank {r}", U, O.col_linear(t["X"].values(), t["A"].values(), r, world), "bf16")
        check(f"Y rank {r}", Y2, O.col_linear(t["X"].values(), t["A"].values(), r, world,
                                              "gelu_tanh"), "bf16")


# ============================================================== the whole MLP backward
@pytest.mark.parametrize("world", [2, 4])
def test_small_mlp_backward(lib, world):
    """Forward with saved pre-activations, then the backward of every rank and the reduce of
    the input-gradient partials, against the oracle's mlp_backward (float64 throughout)."""
    tp, pl = lib
    cfg = small_variant("mlp_bf16_tp4").with_(world=world)
    t = generate(cfg)
    dZ = output_gradient(cfg)
    sh = pl.MLPTrainShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), dev(dZ), world)
    say(f"  small MLP forward + backward world={world} {cfg.tokens}x{cfg.hidden}x{cfg.ffn}")
    sh.forward()
    sh.backward()
    _sync()
    X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
    ref = O.mlp_backward(X, A, B, dZ.values(), world)
    Zref = O.reduce_partials([O.mlp_shard(X, A, B, r, world) for r in range(world)])
    check("Z (forward)", sh.Z, Zref, "bf16")
    check("dX", sh.dX, ref["dX"], "bf16")
    check("dA", sh.dA, ref["dA"], "bf16")
    check("dB", sh.dB, ref["dB"], "bf16")
    fl = cfg.ffn // world
    for r in range(world):
        s = O.mlp_shard_backward(X, A, B, dZ.values(), r, world)
        check(f"dU rank {r}", sh.dU[r], s["dU"], "bf16")
        check(f"dX part rank {r}", sh.dXparts[r], s["dX_part"], "bf16")
        assert sh.dA[:, r * fl:(r + 1) * fl].shape == s["dA"].shape


def test_mlp_backward_deterministic(lib):
    """Two backward passes give identical bits (fixed summation order, no atomics)."""
    tp, pl = lib
    cfg = small_variant("mlp_bf16_tp4")
    t = generate(cfg)
    sh = pl.MLPTrainShard(dev(t["X"]), dev(t["A"]), dev(t["B"]), dev(output_gradient(cfg)),
                          cfg.world)
    say("  MLP backward determinism")
    sh.forward()
    sh.backward()
    first = [x.clone() for x in (sh.dX, sh.dA, sh.dB)]
    sh.backward()
    _sync()
    for a, b in zip(first, (sh.dX, sh.dA, sh.dB)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


# ============================================================== full size
def test_full_mlp_backward(lib):
    """The block workload's MLP shard at full size (X 8192 x 12288, W1 12288 x 49152, W2
    49152 x 12288, 8 ranks), rank 5, launched as the bench launches it.  Every element of
    the saved pre-activation, dU, the dX partial and the rank's dW1 and dW2 blocks against
    the oracle's backward of the shard (6.2 TFLOP of float64)."""
    tp, pl = lib
    cfg = get_config("block_bf16_tp8")
    H, F, P = cfg.hidden, cfg.ffn, cfg.world
    r, fl = 5, F // P
    t = generate(cfg, only={"X", "W1", "W2"})
    dZ = output_gradient(cfg)
    X, A, B = t["X"], t["W1"], t["W2"]
    sh = pl.MLPTrainShard(dev(X), dev(A), dev(B), dev(dZ), P)
    say(f"  full MLP backward rank {r}: forward save, row backward, column backward")
    sh.forward_rank(r)
    sh.backward_row(r)
    sh.backward_col(r)
    _sync()
    say("  full MLP backward: computing the oracle's shard backward")
    ref = O.mlp_shard_backward(X.values(), A.values(), B.values(), dZ.values(), r, P)
    check("U (saved pre-activation)", sh.U[r], ref["U"], "bf16")
    check("dU", sh.dU[r], ref["dU"], "bf16")
    check("dX partial", sh.dXparts[r], ref["dX_part"], "bf16")
    check("dW1 block", sh.dA[:, r * fl:(r + 1) * fl], ref["dA"], "bf16")
    check("dW2 block", sh.dB[r * fl:(r + 1) * fl], ref["dB"], "bf16")
    assert sh.dA.shape == (H, F) and sh.dB.shape == (F, H)


# ============================================================== K tails in the first stages
@pytest.mark.parametrize("kp", [8, 40, 64, 72, 96, 120, 136, 200])
def test_short_contraction_every_layout(lib, kp):
    """Products whose contraction length kp ends inside the first stages, which are loaded
    before the K loop starts: the input-gradient product (B read K-contiguous, with and
    without the GeLU' epilogue), the weight-gradient product (A read M-contiguous) and the
    forward column product (A K-contiguous) must all zero-fill past kp.  Regression test: a
    clobbered condition code once disabled the bound for these stages, so the loads ran on
    into the next row."""
    tp, pl = lib
    rng = _rng(900 + kp)
    seq, kl, N = 40, 256, kp  # dY = dZ[seq, kp] . W_r^T[kp, kl]; the forward uses H = kp
    dZ, W = rng.standard_normal((seq, N)), rng.standard_normal((kl, N)) / np.sqrt(N)
    U, Y = 1.5 * rng.standard_normal((seq, kl)), rng.standard_normal((seq, kl))
    dZd, Wd, Ud, Yd = (dev_values(v, "bf16") for v in (dZ, W, U, Y))
    dZv, Wv, Uv, Yv = (host(t) for t in (dZd, Wd, Ud, Yd))
    for act in (tp.TP_ACT_NONE, tp.TP_ACT_GELU_TANH):
        dY = torch.empty(seq, kl, dtype=torch.bfloat16, device="cuda:0")
        say(f"  short contraction kp={kp} act={act}: input gradient (B^T read K-contiguous)")
        tp.tp_row_linear_backward(dZd, Wd, None, 0, Ud, kl, dY, kl, None, 0, seq, kl, N, 0, 1, act,
                                  0, tp.TP_BF16)
        _sync()
        rdY, _ = O.row_linear_backward(dZv, Yv, Wv, 0, 1, Uv,
                                       "gelu_tanh" if act == tp.TP_ACT_GELU_TANH else "none")
        check(f"dY kp={kp} act={act}", dY, rdY, "bf16")
    # weight gradient with a short sequence: dW[kl, N] = Y[kp, kl]^T . dZ[kp, N]
    Ys, dZs = rng.standard_normal((kp, kl)), rng.standard_normal((kp, 264))
    Ysd, dZsd = dev_values(Ys, "bf16"), dev_values(dZs, "bf16")
    dW = torch.empty(kl, 264, dtype=torch.float32, device="cuda:0")
    say(f"  short contraction kp={kp}: weight gradient (A^T read M-contiguous)")
    tp.tp_row_linear_backward(dZsd, dev_values(rng.standard_normal((kl, 264)), "bf16"), Ysd, kl,
                              None, 0, None, 0, dW, 264, kp, kl, 264, 0, 1, tp.TP_ACT_NONE, 0,
                              tp.TP_BF16)
    _sync()
    check(f"dW kp={kp}", dW, host(Ysd).T @ host(dZsd), "f32")
    # forward column product with H = kp
    X = dev_values(rng.standard_normal((seq, kp)), "bf16")
    Wc = dev_values(rng.standard_normal((kp, 272)) / np.sqrt(kp), "bf16")
    Yc = torch.empty(seq, 272, dtype=torch.bfloat16, device="cuda:0")
    say(f"  short contraction kp={kp}: forward column product")
    tp.tp_col_linear_gelu(X, Wc, Yc, 272, seq, kp, 272, 0, 1, tp.TP_ACT_GELU_TANH, tp.TP_BF16)
    _sync()
    check(f"Y kp={kp}", Yc, O.col_linear(host(X), host(Wc), 0, 1, "gelu_tanh"), "bf16")
