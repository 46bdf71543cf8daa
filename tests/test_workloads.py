"""Host-side input generation: bf16 encoding, determinism, draw order, shapes."""
import numpy as np

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, generate
from workloads.configs import rank_flops, small_variant
from workloads import synth


def test_bf16_round_to_nearest_even():
    def enc(u32):
        return int(f32_to_bf16_bits(np.array([u32], np.uint32).view(np.float32))[0])
    assert enc(0x3F800000) == 0x3F80            # 1.0 exact
    assert enc(0x3F808000) == 0x3F80            # tie, even stays
    assert enc(0x3F818000) == 0x3F82            # tie, odd rounds up
    assert enc(0x3F808001) == 0x3F81            # above half rounds up
    assert enc(0x3F807FFF) == 0x3F80            # below half rounds down
    assert enc(0xBF808001) == 0xBF81            # sign carried
    assert enc(0x3FFF8000) == 0x4000            # carry into the exponent


def test_bf16_decode_exact():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    b = f32_to_bf16_bits(x)
    v = bf16_bits_to_f32(b)
    assert np.all(np.abs(v - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(f32_to_bf16_bits(v), b)


def test_thread_count_does_not_change_values(monkeypatch):
    cfg = small_variant("linear_bf16_tp2").with_(tokens=3000)
    monkeypatch.setattr(synth, "CHUNK_ELEMS", 4096)
    a = generate(cfg, threads=1)
    b = generate(cfg, threads=7)
    for k in a:
        assert np.array_equal(a[k].data, b[k].data)
    c = generate(cfg, only={"W"})
    assert set(c) >= {"W"} and "X" not in c
    assert np.array_equal(c["W"].data, a["W"].data)


def test_deterministic_and_distinct_seeds():
    a = generate(small_variant("mlp_f32_tp2"))
    b = generate(small_variant("mlp_f32_tp2"))
    assert np.array_equal(a["X"].data, b["X"].data)
    c = generate(small_variant("mlp_f32_tp2").with_(seed=5))
    assert not np.array_equal(a["X"].data, c["X"].data)


def test_fan_in_scaling():
    cfg = small_variant("mlp_bf16_tp4").with_(tokens=512, hidden=512, ffn=2048)
    t = generate(cfg)
    assert abs(t["X"].values().std() - 1.0) < 0.02
    assert abs(t["A"].values().std() * np.sqrt(512) - 1.0) < 0.02
    assert abs(t["B"].values().std() * np.sqrt(2048) - 1.0) < 0.02


def test_config_shapes_divide():
    for cfg in CONFIGS.values():
        P = cfg.world
        assert cfg.tokens == cfg.batch * cfg.seq or cfg.kind in ("mlp", "linear")
        if cfg.ffn:
            assert cfg.ffn % P == 0 and (cfg.ffn // P) % 8 == 0
        if cfg.n_heads:
            assert cfg.n_heads % P == 0 and cfg.n_heads * cfg.head_dim == cfg.hidden


def test_rank_flops_block():
    f = rank_flops(CONFIGS["block_bf16_tp8"])
    total = sum(f.values()) / 1e9
    assert abs(total - 3762.4) < 0.1  # GFLOP per rank shard
