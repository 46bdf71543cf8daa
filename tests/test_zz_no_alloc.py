"""The attention-head shard's entry point that allocates nothing (tp_attn_head_shard_noalloc),
against the workspace entry point (tp_attn_head_shard) it shares its kernels with.

Two calls in a row through the C ABI, the second smaller than the first: the full-size rank of
the largest workload served, whose workspace fills the library's static scratch exactly, then
a reduced attention workload.  Each output must be bit-identical to the workspace entry
point's on the same inputs (same kernels, same launch plan), and the reduced one must also
match the float64 oracle within the bf16 tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
from gpu_helpers import bits, check, dev, dev_values, say
from workloads import generate
from workloads.configs import small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp(gpu):
    from megatron_tensor_transformer_linear_amd import tp as mod
    torch.cuda.set_device(0)
    return mod


def _pair(tp, Xn, Wqkv, Wo, batch, seq, H, nh, d, rank, world, causal):
    """(noalloc output, workspace output) fp32 partials of one rank on the same inputs."""
    T = batch * seq
    z_na = torch.full((T, H), float("nan"), dtype=torch.float32, device=Xn.device)
    z_ws = torch.full((T, H), float("nan"), dtype=torch.float32, device=Xn.device)
    tp.tp_attn_head_shard_noalloc(Xn, Wqkv, Wo, z_na, batch, seq, H, nh, d, rank, world,
                                  int(causal), tp.TP_BF16)
    wsb = tp.tp_attn_workspace_bytes(batch, seq, H, nh, d, world, tp.TP_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=Xn.device)
    tp.tp_attn_head_shard(Xn, Wqkv, Wo, z_ws, batch, seq, H, nh, d, rank, world, int(causal),
                          tp.TP_BF16, ws, wsb)
    torch.cuda.synchronize()
    return z_na, z_ws


def test_noalloc_matches_workspace_entry_point(tp):
    dev0 = torch.device("cuda:0")
    # Call 1: one rank (3 of 8) of the block workload at full size, 4 x 2048 tokens,
    # H = 12288, 96 heads: its workspace is exactly the static scratch.  Inputs are seeded
    # bf16 draws on the device (N(0,1) activations, N(0,1/fan_in) weights).
    batch, seq, H, nh, d, world, rank = 4, 2048, 12288, 96, 128, 8, 3
    assert tp.tp_attn_workspace_bytes(batch, seq, H, nh, d, world, tp.TP_BF16) == \
        tp.TP_ATTN_SCRATCH_BYTES
    g = torch.Generator(device=dev0)
    g.manual_seed(71)
    Xn = torch.randn(batch * seq, H, generator=g, device=dev0).to(torch.bfloat16)
    Wqkv = (torch.randn(H, 3 * H, generator=g, device=dev0) / H ** 0.5).to(torch.bfloat16)
    Wo = (torch.randn(H, H, generator=g, device=dev0) / H ** 0.5).to(torch.bfloat16)
    say(f"  noalloc call 1: batch={batch} seq={seq} H={H} heads={nh} world={world} rank={rank}")
    z_na, z_ws = _pair(tp, Xn, Wqkv, Wo, batch, seq, H, nh, d, rank, world, True)
    assert torch.isfinite(z_ws).all()
    n_bad = int(torch.count_nonzero(z_na.view(torch.int32) != z_ws.view(torch.int32)))
    say(f"    full-size rank: bit mismatches {n_bad} / {z_na.numel()}")
    assert n_bad == 0
    del Xn, Wqkv, Wo, z_na, z_ws
    torch.cuda.empty_cache()

    # Call 2: a smaller input, the reduced attention workload (2 x 200 tokens, H = 1024,
    # 8 heads, 4 ranks), rank 1, causal: bit-identical again, and within tolerance of the
    # oracle.
    cfg = small_variant("attn_bf16_tp4")
    t = generate(cfg)
    Wqkv_v = np.hstack([t["Wq"].values(), t["Wk"].values(), t["Wv"].values()])
    Xd, Wqkv_d, Wo_d = dev(t["X"]), dev_values(Wqkv_v, "bf16"), dev(t["Wo"])
    rank = 1
    say(f"  noalloc call 2: {cfg} rank={rank}")
    z_na, z_ws = _pair(tp, Xd, Wqkv_d, Wo_d, cfg.batch, cfg.seq, cfg.hidden, cfg.n_heads,
                       cfg.head_dim, rank, cfg.world, True)
    assert np.array_equal(bits(z_na), bits(z_ws))
    ref = O.attn_head_shard(t["X"].values(), Wqkv_v, t["Wo"].values(), cfg.n_heads,
                            cfg.head_dim, rank, cfg.world, cfg.batch, cfg.seq, True)
    check("noalloc O partial", z_na, ref, "bf16")


def test_noalloc_rejects_beyond_the_scratch(tp):
    """Sizes whose workspace exceeds the static scratch fail before any launch: the output
    keeps its contents."""
    dev0 = torch.device("cuda:0")
    batch, seq, H, nh, d, world = 8, 2048, 12288, 96, 128, 8
    Xn = torch.zeros(16, dtype=torch.bfloat16, device=dev0)
    Z = torch.full((64,), 3.0, dtype=torch.float32, device=dev0)
    with pytest.raises(tp.TPError) as e:
        tp.tp_attn_head_shard_noalloc(Xn, Xn, Xn, Z, batch, seq, H, nh, d, 0, world, 1,
                                      tp.TP_BF16)
    assert e.value.status == tp.TP_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((Z == 3.0).all())
