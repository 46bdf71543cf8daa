"""The five workloads of the tensor-parallel layer shard, plus reduced-size variants.

Shapes follow the statement of a linear layer as Y = X.W with X [seq, H],
W [H, N], Y [seq, N] (pwwt.cn TP article, section 1.1, figure 1).  Weights are
stored [in, out] row-major.  Every weight is drawn from N(0, 1/fan_in), with
fan_in the full (unsharded) input width; activations from N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "mlp" | "linear" | "attn" | "block"
    dtype: str           # "f32" | "bf16"  (io dtype; accumulation is fp32 on the GPU)
    world: int           # simulated tensor-parallel ranks
    seed: int
    tokens: int          # rows T = batch * seq
    hidden: int          # H
    ffn: int = 0         # F (mlp / block)
    n_out: int = 0       # N of the single linear
    batch: int = 1
    seq: int = 0
    n_heads: int = 0
    head_dim: int = 0
    causal: bool = True
    eps: float = 1e-5
    description: str = ""

    def draws(self) -> Tuple[Tuple[str, Tuple[int, int], int], ...]:
        """(name, shape, fan_in) in the fixed draw order; fan_in 0 means N(0,1)."""
        T, H = self.tokens, self.hidden
        if self.kind == "mlp":
            return (("X", (T, H), 0), ("A", (H, self.ffn), H), ("B", (self.ffn, H), self.ffn))
        if self.kind == "linear":
            return (("X", (T, H), 0), ("W", (H, self.n_out), H))
        if self.kind == "attn":
            return (("X", (T, H), 0), ("Wq", (H, H), H), ("Wk", (H, H), H), ("Wv", (H, H), H),
                    ("Wo", (H, H), self.n_heads * self.head_dim))
        if self.kind == "block":
            return (("X", (T, H), 0), ("Wq", (H, H), H), ("Wk", (H, H), H), ("Wv", (H, H), H),
                    ("Wo", (H, H), self.n_heads * self.head_dim),
                    ("W1", (H, self.ffn), H), ("W2", (self.ffn, H), self.ffn))
        raise ValueError(self.kind)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "mlp_f32_tp2": Config(
        name="mlp_f32_tp2", kind="mlp", dtype="f32", world=2, seed=0,
        tokens=64, hidden=256, ffn=1024,
        description="Megatron MLP, fp32, 2 ranks: X[64,256], A[256,1024] column-split, "
                    "GeLU-tanh, B[1024,256] row-split, partials summed to Z[64,256]"),
    "linear_bf16_tp2": Config(
        name="linear_bf16_tp2", kind="linear", dtype="bf16", world=2, seed=1,
        tokens=2048, hidden=4096, n_out=8192,
        description="single linear X[2048,4096].W[4096,8192]: rank-0 column block, and "
                    "2-way row split with fp32 partial sum"),
    "mlp_bf16_tp4": Config(
        name="mlp_bf16_tp4", kind="mlp", dtype="bf16", world=4, seed=2,
        tokens=4096, hidden=4096, ffn=16384, batch=2, seq=2048,
        description="MLP shard H=4096 F=16384 T=4096, 4 ranks, GeLU, 4-part reduce + "
                    "residual + LayerNorm"),
    "attn_bf16_tp4": Config(
        name="attn_bf16_tp4", kind="attn", dtype="bf16", world=4, seed=3,
        tokens=4096, hidden=8192, batch=2, seq=2048, n_heads=64, head_dim=128, causal=True,
        description="attention head shard H=8192, 64 heads x 128, 16 heads per rank, "
                    "batch 2 x seq 2048, causal"),
    "block_bf16_tp8": Config(
        name="block_bf16_tp8", kind="block", dtype="bf16", world=8, seed=7,
        tokens=8192, hidden=12288, ffn=49152, batch=4, seq=2048, n_heads=96, head_dim=128,
        causal=True,
        description="Transformer block shard H=12288, 96 heads x 128, F=49152, 8 ranks "
                    "(12 heads, FFN slice 6144), batch 4 x seq 2048, causal"),
}

ORDER = ("mlp_f32_tp2", "linear_bf16_tp2", "mlp_bf16_tp4", "attn_bf16_tp4", "block_bf16_tp8")


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


def small_variant(name: str) -> Config:
    """Reduced shapes with the same structure: several GEMM tiles plus ragged tails,
    sized so the CPU oracle finishes in about a second."""
    c = CONFIGS[name]
    if name == "mlp_f32_tp2":
        return c.with_(tokens=72, hidden=136, ffn=528)
    if name == "linear_bf16_tp2":
        return c.with_(tokens=300, hidden=272, n_out=784)
    if name == "mlp_bf16_tp4":
        return c.with_(tokens=300, hidden=264, ffn=1088, batch=1, seq=300)
    if name == "attn_bf16_tp4":
        return c.with_(tokens=2 * 200, hidden=1024, batch=2, seq=200, n_heads=8, head_dim=128)
    if name == "block_bf16_tp8":
        return c.with_(tokens=2 * 136, hidden=2048, ffn=4096, batch=2, seq=136, n_heads=16,
                       head_dim=128)
    raise KeyError(name)


def rank_flops(cfg: Config) -> Dict[str, float]:
    """Algorithmic flops of one rank's shard, per stage (2 flops per multiply-add;
    causal attention counts only the visible (query, key) pairs)."""
    P, T, H = cfg.world, cfg.tokens, cfg.hidden
    out: Dict[str, float] = {}
    if cfg.kind in ("mlp", "block"):
        F = cfg.ffn
        out["mlp_col"] = 2.0 * T * H * (F // P)
        out["mlp_row"] = 2.0 * T * (F // P) * H
    if cfg.kind == "linear":
        out["col"] = 2.0 * T * H * (cfg.n_out // P)
        out["row"] = 2.0 * T * (H // P) * cfg.n_out
    if cfg.kind in ("attn", "block"):
        hl = cfg.n_heads // P
        d = cfg.head_dim
        out["qkv"] = 2.0 * T * H * (3 * hl * d)
        S = cfg.seq
        pairs = S * (S + 1) / 2 if cfg.causal else S * S
        out["attn_core"] = 4.0 * d * pairs * hl * cfg.batch
        out["o_proj"] = 2.0 * T * (hl * d) * H
    return out



def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "f32": 4}[dtype]


def tensor_bytes(rows: int, cols: int, dtype: str) -> int:
    """Bytes of a dense [rows, cols] tensor."""
    return rows * cols * elem_bytes(dtype)


def reduce_bytes(rows: int, hidden: int, n_parts: int, dtype: str, residual: bool,
                 h_out: bool, y_out: bool, parts_dtype: str = "f32") -> int:
    """Algorithmic HBM bytes of one reduce + residual + LayerNorm pass: every partial
    (fp32, or bf16 for the bf16-partial variant) and the residual read once, every output
    written once (gamma and beta, a single row each, are not counted)."""
    b = n_parts * tensor_bytes(rows, hidden, parts_dtype)
    b += (int(residual) + int(h_out) + int(y_out)) * tensor_bytes(rows, hidden, dtype)
    return b
