#!/usr/bin/env python3
"""Throughput of the tensor-parallel Transformer-block shard on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: the block
workload H=12288, 96 heads x 128, F=49152, 8 simulated tensor-parallel ranks (12 heads and
an FFN slice of 6144 each), batch 4 x seq 2048, causal, bf16 with fp32 accumulation:

    xn = LN(X)                                   reduce kernel, no partials
    for r in 0..7: attention-head shard of r     QKV GEMM, attention, O GEMM -> fp32 partial
    h, hn = X + sum_r partials, LN(h)            reduce + residual + LayerNorm
    for r in 0..7: MLP shard of r                column GEMM + GeLU, row GEMM -> fp32 partial
    out = h + sum_r partials                     reduce + residual

Inputs are generated and resident in HBM before the timed region.  `value` is the whole
step's algorithmic flops (all 8 ranks' shards) divided by the measured step time, in
TFLOP/s, over steps run back to back.  Per-kernel durations come from HIP events recorded on
the launch stream inside the timed region; the roofline object reports the kernel with the
most time per step (one of the two MLP GEMMs), `rooflines` both.  The graphics and memory
clocks are sampled through amdsmi over a separate ~6 s run of the same steps, and the
fractions of peak are also given at that graphics clock, and against the matrix-core rate the
device sustains with no memory traffic at all in the same power state (`mfma_ceiling`: a
calibration loop of MFMAs on random operands).  A cold-cache pass then times every
stage again after reading 512 MiB of scratch (twice the 256 MB Infinity Cache) just before
it, so nothing it reads is cached (`stages[*].cold_*`).  The CPU baseline times the float64
oracle on a bounded row sample of the same workload on this host, and the full oracle of each
other workload.  After the timed steps, the sequence-parallel form of the epilogue (each
rank's reduce-scatter of its 1024 rows) and the backward pass of the MLP pair (the four
gradient products of every rank and the reduce of the input-gradient partials, with those
partials also stored in bf16 and reduced; --no-backward skips it) are timed on their own and reported beside the step, outside `value`, and so is the
same step with each epilogue's reduce folded into the row-parallel products (one fp32 running
sum instead of 8 stacked partials; --no-fold skips it) and with the 8 partials stored in bf16
(--no-bf16-partials skips it).  The other workloads of the path (the
fp32 MLP, the single linear, the bf16 MLP shard and the attention-head shard) are timed the
same way and reported per rank under `other_workloads` (--no-workloads skips them).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import generate, get_config  # noqa: E402
from workloads.configs import rank_flops, reduce_bytes  # noqa: E402

WORKLOAD = "block_bf16_tp8"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
PEAK_F32_MFMA_TFLOPS = 157.3  # dense fp32 MFMA


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_block_bf16_tp8_hbm_traffic.md")
FLUSH_MIB = 512  # scratch read before each cold-cache stage: 2x the 256 MB Infinity Cache


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(role: str):
    """HBM bytes per launch of one GEMM role ("mlp_col", "mlp_row") from the committed counter
    summary (lines `traffic_bytes_per_launch.<role>: N`), or None when the kernel sources no
    longer hash to the digest the counters were taken at."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE).read().splitlines():
            if ": " in line:
                k, v = line.split(": ", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in kv["kernel_sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv["kernel_sources_sha256"]:
            return None
        return int(kv["traffic_bytes_per_launch." + role])
    except (OSError, KeyError, ValueError):
        return None


class ClockSampler:
    """Samples the GPU's graphics clock (mean over its XCDs), memory clock and socket power
    through amdsmi's GPU metrics every `period` seconds on a thread, between start() and
    stop().  amdsmi reads the driver's metrics table; it makes no HIP call.  The firmware
    refreshes that table far less often than every step, so only samples whose firmware
    timestamp changed are kept, and the bench samples a run of several seconds (clock_leg).
    Any failure (no amdsmi, no matching device) leaves the summary's `error` set instead of
    clocks."""

    def __init__(self, period: float = 0.05):
        import threading
        self.period, self.samples, self.error = period, [], None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            import torch
            self._amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            want = None
            try:
                p = torch.cuda.get_device_properties(0)
                want = (int(p.pci_domain_id), int(p.pci_bus_id), int(p.pci_device_id))
            except Exception:  # noqa: BLE001 - older torch: no PCI ids
                pass
            for h in handles:
                if want is None:
                    break
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._handle = h
            if self._handle is None and len(handles) == 1:
                self._handle = handles[0]
            if self._handle is None:
                self.error = f"no amdsmi device matched ({len(handles)} visible)"
        except Exception as e:  # noqa: BLE001
            self.error = f"amdsmi unavailable: {e}"

    @staticmethod
    def _num(v):
        return float(v) if isinstance(v, (int, float)) and not isinstance(v, bool) else None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        gfx = [self._num(v) for v in (m.get("current_gfxclks") or [])]
        gfx = [v for v in gfx if v]
        if not gfx and self._num(m.get("current_gfxclk")):
            gfx = [self._num(m["current_gfxclk"])]
        return (sum(gfx) / len(gfx) if gfx else None, self._num(m.get("current_uclk")),
                self._num(m.get("current_socket_power")), m.get("firmware_timestamp"))

    def _run(self):
        last = None
        while not self._stop.wait(self.period):
            try:
                x = self._read()
            except Exception as e:  # noqa: BLE001
                self.error = f"amdsmi read failed: {e}"
                return
            if x[3] is None or x[3] != last:  # a refreshed table (or no timestamp to tell)
                self.samples.append(x[:3])
                last = x[3]

    def start(self):
        if self._handle is None:
            return
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self) -> dict:
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        out = {"source": "amdsmi GPU metrics (current_gfxclks averaged over the XCDs, "
                         f"current_uclk, current_socket_power), polled every "
                         f"{self.period * 1e3:.0f} ms, one sample per firmware refresh",
               "samples": len(self.samples)}
        if self.error:
            out["error"] = self.error

        def summary(i):
            v = sorted(x[i] for x in self.samples if x[i] is not None)
            if not v:
                return None
            return {"median": v[len(v) // 2], "mean": round(sum(v) / len(v), 1),
                    "min": v[0], "max": v[-1]}
        if self.samples:
            out["sclk_mhz"] = summary(0)
            out["mclk_mhz"] = summary(1)
            out["socket_power_w"] = summary(2)
        return out


class CacheFlush:
    """Reads FLUSH_MIB MiB of scratch (one reduction kernel) on the current stream, evicting
    everything a following kernel reads from the L2s and the 256 MB Infinity Cache.  A read
    sweep leaves the caches holding clean lines: a write sweep (a fill) would leave up to
    256 MB of dirty lines whose write-back then runs during the timed stage and is charged
    to it (it doubled the pre-LayerNorm's cold time)."""

    def __init__(self, dev, mib: int = FLUSH_MIB):
        import torch
        self.buf = torch.ones(mib << 18, dtype=torch.float32, device=dev)
        self.sink = torch.zeros((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def cpu_baseline(cfg, t, qkv_vals) -> dict:
    """The oracle as it stands, on a bounded row sample of the same block workload."""
    import oracle.tp_oracle as O
    S = cfg.seq
    per_seq = np.unique(np.concatenate([np.linspace(0, S - 1, 256).astype(np.int64), [S - 1]]))
    rows = np.concatenate([b * S + per_seq for b in range(cfg.batch)])
    g, b = t["gamma"].values(), t["beta"].values()
    args = (t["X"].values(), qkv_vals, t["Wo"].values(), t["W1"].values(), t["W2"].values(),
            g, b, g, b)
    t0 = time.perf_counter()
    O.block_shard(*args, n_heads=cfg.n_heads, head_dim=cfg.head_dim, world=cfg.world,
                  batch=cfg.batch, seq=S, causal=True, eps=cfg.eps, rows=rows,
                  keep_partials=False)
    dt = time.perf_counter() - t0
    # algorithmic flops the sample needs: K and V over the causal prefix of every rank,
    # Q, attention and O for the sampled rows, and the MLP of every rank for those rows.
    H, P, d = cfg.hidden, cfg.world, cfg.head_dim
    hl = cfg.n_heads // P
    nb = hl * d
    R = len(rows)
    pos = rows % S
    kv_tokens = cfg.batch * (int(pos.max()) + 1)
    per_rank = (2.0 * kv_tokens * H * 2 * nb + 2.0 * R * H * nb
                + sum(4.0 * d * (int(i) + 1) * hl for i in pos) + 2.0 * R * nb * H
                + 2.0 * 2.0 * R * H * (cfg.ffn // P))
    flops = per_rank * P
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": (f"float64 oracle of the whole 8-rank block for {R} query rows "
                       f"({len(per_seq)} positions spread over 0..{S - 1} in each of the "
                       f"{cfg.batch} sequences; keys/values over the full causal prefixes): "
                       f"{flops / 1e9:.0f} GFLOP in {dt:.1f} s; its matrix products are "
                       "numpy float64 BLAS")}


def mlp_backward_leg(cfg, t, blk, stream) -> dict:
    """Backward of the block's MLP pair (outside the timed forward step): every rank's four
    backward products, dY = dZ.W2_r^T with GeLU' fused, dW2_r = Y_r^T.dZ, dX_r = dU_r.W1_r^T,
    dW1_r = X^T.dU_r, then the reduce of the 8 input-gradient partials.  One untimed pass,
    then two timed passes; each kind of product runs for the 8 ranks back to back and is timed
    as a group with HIP events on its stream at the group boundaries (per launch: the group's
    time over 8).  After each pass, the dX partials stored in bf16 and their reduce are timed
    the same way; pass_bf16_dx_ms is the pass with those two groups swapped in."""
    import torch
    from megatron_tensor_transformer_linear_amd import pipeline as pl
    from workloads import output_gradient

    dev = torch.device("cuda:0")
    dZ = pl.to_device(output_gradient(cfg).data, "bf16", dev)
    trn = pl.MLPTrainShard(blk.X, blk.W1, blk.W2, dZ, cfg.world)
    trn.forward()  # saves U_r and Y_r of every rank
    # The same dX partials stored in bf16 and their reduce, from trn's dU (timed after the pass).
    half = pl.MLPTrainShard(blk.X, blk.W1, blk.W2, dZ, cfg.world, bf16_dx_partials=True)
    half.dU = trn.dU
    legs = {"dY": lambda r: trn.backward_row(r, True, False),
            "dW2": lambda r: trn.backward_row(r, False, True),
            "dX_part": lambda r: trn.backward_col(r, True, False),
            "dW1": lambda r: trn.backward_col(r, False, True)}
    ev = {k: [] for k in list(legs) + ["reduce_dX", "pass", "dX_part_bf16", "reduce_dX_bf16"]}
    # Each product runs for all ranks back to back (rank r's dX and dW1 read its dU_r, which
    # its dY product wrote in an earlier group), with events only at the group boundaries.
    for it in range(3):
        s0 = prev = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for k, fn in legs.items():
            for r in range(cfg.world):
                fn(r)
            e_ = torch.cuda.Event(enable_timing=True)
            e_.record(stream)
            if it > 0:
                ev[k].append((prev, e_))
            prev = e_
        trn.reduce_dx()
        e_ = torch.cuda.Event(enable_timing=True)
        e_.record(stream)
        if it > 0:
            ev["reduce_dX"].append((prev, e_))
            ev["pass"].append((s0, e_))
        prev = e_
        for r in range(cfg.world):
            half.backward_col(r, True, False)
        e_ = torch.cuda.Event(enable_timing=True)
        e_.record(stream)
        if it > 0:
            ev["dX_part_bf16"].append((prev, e_))
        prev = e_
        half.reduce_dx()
        e_ = torch.cuda.Event(enable_timing=True)
        e_.record(stream)
        if it > 0:
            ev["reduce_dX_bf16"].append((prev, e_))
    torch.cuda.synchronize()
    T, H, fl = cfg.tokens, cfg.hidden, cfg.ffn // cfg.world
    gemm_flops = 2.0 * T * H * fl  # each of the four products
    out = {"what": "backward of the MLP pair, 8 ranks: dY (NT, GeLU' fused), dW2 (TN), "
                   "dX partial (NT), dW1 (TN), reduce of the dX partials",
           "gemm_gflop_per_rank": round(4 * gemm_flops / 1e9, 1)}
    for k in legs:
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[k]])) / cfg.world
        out[k] = {"avg_ms": round(ms, 4), "tflops": round(gemm_flops / ms / 1e9, 1)}
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev["reduce_dX"]]))
    nbytes = reduce_bytes(T, H, cfg.world, "bf16", residual=False, h_out=True, y_out=False)
    out["reduce_dX"] = {"avg_ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                        "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev["pass"]]))
    out["pass_ms"] = round(ms, 3)
    out["pass_tflops"] = round(cfg.world * 4 * gemm_flops / ms / 1e9, 1)
    # the variant with the dX partials exchanged in bf16 (the fp32 pass above is the measure)
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev["dX_part_bf16"]])) / cfg.world
    out["dX_part_bf16"] = {"avg_ms": round(ms, 4), "tflops": round(gemm_flops / ms / 1e9, 1)}
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev["reduce_dX_bf16"]]))
    nbytes = reduce_bytes(T, H, cfg.world, "bf16", residual=False, h_out=True, y_out=False,
                          parts_dtype="bf16")
    out["reduce_dX_bf16"] = {"avg_ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                             "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    out["pass_bf16_dx_ms"] = round(out["pass_ms"] + cfg.world * (out["dX_part_bf16"]["avg_ms"]
                                   - out["dX_part"]["avg_ms"]) + out["reduce_dX_bf16"]["avg_ms"]
                                   - out["reduce_dX"]["avg_ms"], 3)
    del trn, half
    return out


def folded_block_leg(cfg, blk, stream, steps: int, variant: str = "fold") -> dict:
    """The same block step in one of the two variants of the exchange, with the same weights
    and inputs as the timed step:
      fold:   the reduce folded into the row-parallel products (each rank's output projection
              and MLP row GEMM add their partial to one fp32 running sum in ascending rank
              order; the epilogues then read one partial instead of 8); the outputs are
              bit-identical to the timed step's;
      bf16:   the 8 partials stored in bf16 (each rounded once), the epilogues reading half
              the bytes; the outputs differ from the timed step's by that rounding."""
    import torch
    from megatron_tensor_transformer_linear_amd import pipeline as pl
    from workloads.configs import rank_flops, reduce_bytes

    fold = variant == "fold"
    fb = pl.BlockShard(blk.X, blk.Wqkv, blk.Wo, blk.W1, blk.W2, blk.g1, blk.b1, blk.g2, blk.b2,
                       cfg.world, cfg.batch, cfg.seq, cfg.n_heads, cfg.head_dim, True, cfg.eps,
                       fold=fold, bf16_partials=not fold)
    ev = {k: [] for k in LAUNCHES}
    step = stage_step(cfg, fb, stream, ev)

    step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fl = rank_flops(cfg)
    step_flops = cfg.world * sum(fl.values())
    T, H = cfg.tokens, cfg.hidden
    n_parts, pdt = (1, "f32") if fold else (cfg.world, "bf16")
    r1 = reduce_bytes(T, H, n_parts, "bf16", residual=True, h_out=True, y_out=True, parts_dtype=pdt)
    r2 = reduce_bytes(T, H, n_parts, "bf16", residual=True, h_out=True, y_out=False, parts_dtype=pdt)

    def avg_ms(key):  # per launch
        return float(np.mean([s.elapsed_time(e) for s, e in ev[key]])) / LAUNCHES[key]

    out = {
        "what": ("the block step with each epilogue's reduce folded into the row-parallel "
                 "products' epilogues (one fp32 running sum, ranks added in ascending order); "
                 "bit-identical outputs" if fold else
                 "the block step with every rank's partial stored in bf16 (the exchanged "
                 "activation at 2 bytes per element), summed in fp32; outputs differ from the "
                 "timed step's by the partials' rounding"),
        "steps": steps,
        "ms_per_step": round(elapsed / steps * 1e3, 3),
        "tflops": round(step_flops * steps / elapsed / 1e12, 2),
        "attn_avg_ms": round(avg_ms("attn"), 4),
        "mlp_row_avg_ms": round(avg_ms("mlp_row"), 4),
        "mlp_row_tflops": round(fl["mlp_row"] / avg_ms("mlp_row") / 1e9, 1),
        "reduce1_ms": round(avg_ms("reduce1"), 4),
        "reduce1_gbs": round(r1 / avg_ms("reduce1") / 1e6, 1),
        "reduce2_ms": round(avg_ms("reduce2"), 4),
        "reduce2_gbs": round(r2 / avg_ms("reduce2") / 1e6, 1),
    }
    del fb
    torch.cuda.empty_cache()
    return out


# Calls per step of each stage: the attention-head shard, the column GEMM and the row GEMM run
# once per simulated rank, the LayerNorm and the two reduces once.
LAUNCHES = {"pre_ln": 1, "attn": 8, "reduce1": 1, "mlp_col": 8, "mlp_row": 8, "reduce2": 1}


def rank_shard(fl: dict, stages: dict, sclk_ghz=None) -> dict:
    ms = stages["attn"]["avg_ms"] + stages["mlp_col"]["avg_ms"] + stages["mlp_row"]["avg_ms"]
    tf = sum(fl.values()) / ms / 1e9
    out = {"ms": round(ms, 4), "gflop": round(sum(fl.values()) / 1e9, 1), "tflops": round(tf, 1),
           "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    if sclk_ghz:
        out["pct_at_measured_sclk"] = round(100 * tf / (PEAK_BF16_TFLOPS * sclk_ghz / 2.4), 2)
    return out


def stage_step(cfg, blk, stream, ev):
    """One block step as stages, with a HIP event at each stage boundary when recording: the
    pre-LayerNorm, the 8 ranks' attention-head shards, the first reduce, the 8 ranks' MLP
    column GEMMs, their 8 row GEMMs, the second reduce.  The MLP runs all ranks' column
    products, then all their row products (the ranks are independent; each rank's hidden
    block stays in its own buffer).  An event recorded between two kernels holds the second
    back for several microseconds on MI355X (a step with an event pair around every call had
    about 270 us of idle gaps), so a step records 7 events: each stage's interval covers its
    launches back to back, and a per-launch time is that interval over the launch count."""
    import torch
    assert cfg.world == LAUNCHES["attn"]
    stages = (("pre_ln", lambda: blk.pre_ln()),
              ("attn", lambda: [blk.attn(r) for r in range(cfg.world)]),
              ("reduce1", lambda: blk.reduce1()),
              ("mlp_col", lambda: [blk.mlp_col(r) for r in range(cfg.world)]),
              ("mlp_row", lambda: [blk.mlp_row(r) for r in range(cfg.world)]),
              ("reduce2", lambda: blk.reduce2()))

    def step(record: bool):
        prev = None
        if record:
            prev = torch.cuda.Event(enable_timing=True)
            prev.record(stream)
        for key, fn in stages:
            fn()
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev[key].append((prev, e))
                prev = e
    return step


def clock_leg(step, ms_per_step: float, seconds: float = 6.0) -> dict:
    """The block step back to back for about `seconds` while the clocks are sampled; the
    first second (the clock settling under load) is left out of the summary."""
    import torch
    n = max(1, int(seconds * 1e3 / ms_per_step))
    sampler = ClockSampler()
    if sampler.error:
        return {"error": sampler.error}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step(False)
    # sample only once the queue is full and the first second has passed
    while time.perf_counter() - t0 < 1.0:
        time.sleep(0.01)
    sampler.start()
    torch.cuda.synchronize()
    out = sampler.stop()
    out["steps"] = n
    out["window_s"] = round(time.perf_counter() - t0 - 1.0, 2)
    return out


def cold_stages(cfg, blk, stream, flush, n_steps: int) -> dict:
    """Each stage of the block step after a cache flush: per step, for every stage in order,
    FLUSH_MIB MiB of scratch are read, then the stage runs between two events.  The stage's
    first launch therefore finds nothing of its operands cached (later launches of a stage,
    the 8 ranks back to back, see what the earlier ones left, as in the step).  Returns the
    per-launch milliseconds of each stage, averaged over n_steps."""
    import torch
    stages = (("pre_ln", lambda: blk.pre_ln()),
              ("attn", lambda: [blk.attn(r) for r in range(cfg.world)]),
              ("reduce1", lambda: blk.reduce1()),
              ("mlp_col", lambda: [blk.mlp_col(r) for r in range(cfg.world)]),
              ("mlp_row", lambda: [blk.mlp_row(r) for r in range(cfg.world)]),
              ("reduce2", lambda: blk.reduce2()))
    ev = {k: [] for k, _ in stages}
    for _ in range(n_steps):
        for key, fn in stages:
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[key].append((a, b))
    torch.cuda.synchronize()
    return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) / LAUNCHES[k]
            for k, v in ev.items()}


def oracle_full(cfg, t) -> dict:
    """The float64 oracle of a whole workload (every rank, and the reduce), timed on this
    host's cores.  Its matrix products are numpy's float64 BLAS (threaded over the host's
    cores); everything else is elementwise numpy."""
    import oracle.tp_oracle as O
    P = cfg.world
    t0 = time.perf_counter()
    if cfg.kind == "mlp":
        X, A, B = t["X"].values(), t["A"].values(), t["B"].values()
        parts = [O.mlp_shard(X, A, B, r, P) for r in range(P)]
        if cfg.dtype == "bf16":
            O.reduce_residual_layernorm(parts, X, t["gamma"].values(), t["beta"].values(), cfg.eps)
        else:
            O.reduce_partials(parts)
    elif cfg.kind == "linear":
        X, W = t["X"].values(), t["W"].values()
        O.col_linear(X, W, 0, P)
        O.reduce_partials([O.row_linear_partial(X, W, r, P) for r in range(P)])
    else:
        X = t["X"].values()
        qkv = np.hstack([t["Wq"].values(), t["Wk"].values(), t["Wv"].values()])
        Wo = t["Wo"].values()
        O.reduce_partials([O.attn_head_shard(X, qkv, Wo, cfg.n_heads, cfg.head_dim, r, P,
                                             cfg.batch, cfg.seq, cfg.causal) for r in range(P)])
    return {"seconds": time.perf_counter() - t0}


def other_workloads_leg(dev, steps: int = 5, flush=None, cpu: bool = True) -> dict:
    """The other workloads of this path, each on its own and outside `value`: the fp32 MLP
    (2 ranks, 64 tokens), the single linear (rank 0's column block and both row partials),
    the bf16 MLP shard (4 ranks, 4096 tokens) and the attention-head shard (4 ranks, 16 heads
    each).  Each stage runs for every rank back to back, with HIP events only at the stage
    boundaries; 1 untimed step, then `steps` timed ones.  Per-rank times are a stage's
    interval over its rank count.  With `flush`, the warm pass starts behind a few reads of
    the scratch (so the host has queued its launches before the GPU reaches them), and a
    second pass times each stage again with the scratch read just before it (the `cold_`
    figures; the others are warm: each stage follows the previous one).  With `cpu`, the float64 oracle of the whole workload is timed
    on this host (`cpu_oracle`)."""
    import torch
    from megatron_tensor_transformer_linear_amd import pipeline as pl

    stream = torch.cuda.current_stream()

    def run(stages, n_steps, cold=False):
        ev = {k: [] for k, _ in stages}
        if not cold and flush is not None:
            # A head start: the GPU reads the scratch while the host queues the launches
            # below, so the warm intervals of microsecond kernels (the fp32 MLP) measure the
            # GPU and not the rate at which the host launches them.
            for _ in range(16):
                flush()
        for it in range(n_steps + 1):
            prev = torch.cuda.Event(enable_timing=True)
            prev.record(stream)
            for key, fn in stages:
                if cold:
                    flush()
                    prev = torch.cuda.Event(enable_timing=True)
                    prev.record(stream)
                fn()
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                if it > 0:
                    ev[key].append((prev, e))
                prev = e
        torch.cuda.synchronize()
        return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}

    def timed(stages):
        """(warm, cold) stage milliseconds; cold is None without a flush."""
        return run(stages, steps), (run(stages, steps, cold=True) if flush else None)

    out = {}
    for name in ("mlp_f32_tp2", "linear_bf16_tp2", "mlp_bf16_tp4", "attn_bf16_tp4"):
        cfg = get_config(name)
        t = generate(cfg)
        up = lambda a: pl.to_device(a.data, cfg.dtype, dev)  # noqa: E731
        fl = rank_flops(cfg)
        P, T, H = cfg.world, cfg.tokens, cfg.hidden
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
        if cfg.kind == "mlp":
            sh = pl.MLPShard(up(t["X"]), up(t["A"]), up(t["B"]), P, cfg.dtype,
                             gamma=up(t["gamma"]), beta=up(t["beta"]), eps=cfg.eps,
                             residual_ln=cfg.dtype == "bf16")
            ms, cms = timed((("column", lambda: [sh.column(r) for r in range(P)]),
                             ("row", lambda: [sh.row(r) for r in range(P)]),
                             ("reduce", sh.reduce)))
            shard_ms = (ms["column"] + ms["row"]) / P
            rb = reduce_bytes(T, H, P, cfg.dtype, residual=sh.residual_ln, h_out=True,
                              y_out=sh.residual_ln) if cfg.dtype == "bf16" else \
                reduce_bytes(T, H, P, "f32", residual=False, h_out=True, y_out=False)
            entry = {"shard_us_per_rank": round(shard_ms * 1e3, 2),
                     "column_us": round(ms["column"] / P * 1e3, 2),
                     "row_us": round(ms["row"] / P * 1e3, 2),
                     "tflops_per_rank": round((fl["mlp_col"] + fl["mlp_row"]) / shard_ms / 1e9, 1),
                     "reduce_us": round(ms["reduce"] * 1e3, 2),
                     "reduce_gbs": round(rb / ms["reduce"] / 1e6, 1)}
            if cms:
                entry.update({"cold_column_us": round(cms["column"] / P * 1e3, 2),
                              "cold_row_us": round(cms["row"] / P * 1e3, 2),
                              "cold_reduce_us": round(cms["reduce"] * 1e3, 2),
                              "cold_reduce_gbs": round(rb / cms["reduce"] / 1e6, 1),
                              "cold_reduce_hbm_frac": round(rb / cms["reduce"] / 1e6 /
                                                            PEAK_HBM_GBS, 3)})
            entry["reduce_hbm_frac"] = round(rb / ms["reduce"] / 1e6 / PEAK_HBM_GBS, 3)
        elif cfg.kind == "linear":
            sh = pl.LinearShard(up(t["X"]), up(t["W"]), P, cfg.dtype, col_ranks=(0,))
            ms, cms = timed((("column", lambda: sh.column(0)),
                             ("row", lambda: [sh.row(r) for r in range(P)]),
                             ("reduce", sh.reduce)))
            rb = reduce_bytes(T, cfg.n_out, P, "f32", residual=False, h_out=True, y_out=False)
            entry = {"column_rank0_us": round(ms["column"] * 1e3, 2),
                     "column_tflops": round(fl["col"] / ms["column"] / 1e9, 1),
                     "row_us_per_rank": round(ms["row"] / P * 1e3, 2),
                     "row_tflops": round(fl["row"] / (ms["row"] / P) / 1e9, 1),
                     "reduce_us": round(ms["reduce"] * 1e3, 2),
                     "reduce_gbs": round(rb / ms["reduce"] / 1e6, 1),
                     "reduce_hbm_frac": round(rb / ms["reduce"] / 1e6 / PEAK_HBM_GBS, 3)}
            if cms:
                entry.update({"cold_column_rank0_us": round(cms["column"] * 1e3, 2),
                              "cold_row_us_per_rank": round(cms["row"] / P * 1e3, 2),
                              "cold_reduce_us": round(cms["reduce"] * 1e3, 2),
                              "cold_reduce_gbs": round(rb / cms["reduce"] / 1e6, 1),
                              "cold_reduce_hbm_frac": round(rb / cms["reduce"] / 1e6 /
                                                            PEAK_HBM_GBS, 3)})
            shard_ms = ms["column"]
            entry["tflops_per_rank"] = entry["column_tflops"]
        else:
            qkv = np.ascontiguousarray(np.hstack([t["Wq"].data, t["Wk"].data, t["Wv"].data]))
            sh = pl.AttnShard(up(t["X"]), pl.to_device(qkv, "bf16", dev), up(t["Wo"]), P,
                              cfg.batch, cfg.seq, cfg.n_heads, cfg.head_dim, cfg.causal)
            ms, cms = timed((("shard", lambda: [sh.rank(r) for r in range(P)]),
                             ("reduce", sh.reduce)))
            shard_ms = ms["shard"] / P
            rb = reduce_bytes(T, H, P, "f32", residual=False, h_out=True, y_out=False)
            entry = {"shard_us_per_rank": round(shard_ms * 1e3, 2),
                     "tflops_per_rank": round((fl["qkv"] + fl["attn_core"] + fl["o_proj"]) /
                                              shard_ms / 1e9, 1),
                     "sum_of_partials_us": round(ms["reduce"] * 1e3, 2),
                     "sum_of_partials_gbs": round(rb / ms["reduce"] / 1e6, 1)}
            if cms:
                entry.update({"cold_shard_us_per_rank": round(cms["shard"] / P * 1e3, 2),
                              "cold_sum_of_partials_us": round(cms["reduce"] * 1e3, 2),
                              "cold_sum_of_partials_gbs": round(rb / cms["reduce"] / 1e6, 1)})
        entry["pct_of_peak"] = round(100 * entry["tflops_per_rank"] / peak, 2)
        if cpu:
            gpu_ms = sum(ms.values())  # every rank and the reduce, warm
            flops = P * sum(fl.values()) if cfg.kind != "linear" else fl["col"] + P * fl["row"]
            o = oracle_full(cfg, t)
            entry["cpu_oracle"] = {
                "kind": "oracle", "cores": len(os.sched_getaffinity(0)),
                "seconds": round(o["seconds"], 3),
                "value": round(flops / o["seconds"] / 1e12, 4), "unit": "TFLOP/s",
                "sample": (f"the whole workload, every rank and the reduce ({flops / 1e9:.1f} "
                           "GFLOP), float64; its matrix products are numpy float64 BLAS"),
                "gpu_ms_same_work": round(gpu_ms, 4),
                "gpu_speedup": round(o["seconds"] * 1e3 / gpu_ms, 1)}
        out[name] = entry
        del sh, t
        torch.cuda.empty_cache()
        log(f"workload {name} timed")
    return out


def mfma_ceiling_leg(dev, a_src, b_src, launches: int = 3, iters: int = 100000) -> dict:
    """The matrix-core rate the device sustains with no memory traffic at all: the calibration
    kernel (calib/mfma_rate.hip: back-to-back bf16 MFMAs whose operands are fragments of the
    workload's own X and W1, two waves per SIMD) timed with HIP events right after the clock
    run, in the same power state.  Under the socket power limit this, not the 2.5 PFLOP/s
    spec, bounds what a GEMM on these operands can reach here; the rooflines report their
    fraction of it."""
    import ctypes
    import torch
    from megatron_tensor_transformer_linear_amd._build import CALIB_LIB_PATH
    if not os.path.exists(CALIB_LIB_PATH):
        return {"error": f"{CALIB_LIB_PATH} not built"}
    lib = ctypes.CDLL(CALIB_LIB_PATH)
    lib.tp_calib_mfma_loop.restype = ctypes.c_int
    lib.tp_calib_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    nbytes = min(a_src.numel() * a_src.element_size(), b_src.numel() * b_src.element_size())
    nbytes -= nbytes % 16
    lib.tp_calib_mfma_flops.restype = ctypes.c_double
    lib.tp_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus  # two 4-wave workgroups per CU: two waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rates = []
    for i in range(launches + 1):
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        rc = lib.tp_calib_mfma_loop(ctypes.c_void_p(a_src.data_ptr()),
                                    ctypes.c_void_p(b_src.data_ptr()), nbytes,
                                    ctypes.c_void_p(out.data_ptr()), blocks,
                                    iters if i else iters // 10, ctypes.c_void_p(stream.cuda_stream))
        e_.record(stream)
        if rc != 0:
            return {"error": f"tp_calib_mfma_loop returned {rc}"}
        torch.cuda.synchronize()
        if i:  # the first, shorter launch is a warm-up
            rates.append(lib.tp_calib_mfma_flops(blocks, iters) / (s_.elapsed_time(e_) * 1e-3) / 1e12)
    rates.sort()
    return {"what": "bf16 MFMA loop, operands taken from the workload's X and W1, no memory "
                    "traffic, two waves per SIMD (calib/mfma_rate.hip), timed right after the "
                    "clock run",
            "tflops": round(rates[len(rates) // 2], 1), "tflops_all": [round(r, 1) for r in rates],
            "frac_of_spec": round(rates[len(rates) // 2] / PEAK_BF16_TFLOPS, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement of the MLP pair")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the measurement of the other workloads (fp32 MLP, single linear, "
                         "bf16 MLP shard, attention-head shard)")
    ap.add_argument("--no-fold", action="store_true",
                    help="skip the measurement of the step with folded reduces")
    ap.add_argument("--no-bf16-partials", action="store_true",
                    help="skip the measurement of the step with bf16 partials")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (each stage after a 512 MiB scratch read)")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the GPU clocks through amdsmi during the timed steps")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the matrix-core rate calibration run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain copy kernel over MIB mebibytes (reads and writes "
                         "MIB each), the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the tensor-parallel ranks are simulated in turn "
              "on that GPU, and no multi-GPU path exists in this library.", file=sys.stderr)
        return 2

    import torch
    from megatron_tensor_transformer_linear_amd import pipeline as pl
    from megatron_tensor_transformer_linear_amd import tp

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 18  # float32 elements in MIB mebibytes
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes MIB MiB each
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration kernel over {args.copy_calibration} MiB done")
    cfg = get_config(WORKLOAD)
    t0 = time.time()
    t = generate(cfg)
    qkv_bits = np.ascontiguousarray(np.hstack([t["Wq"].data, t["Wk"].data, t["Wv"].data]))
    log(f"inputs generated in {time.time() - t0:.1f} s")

    def up(a):
        return pl.to_device(a, "bf16", dev)

    blk = pl.BlockShard(up(t["X"].data), up(qkv_bits), up(t["Wo"].data), up(t["W1"].data),
                        up(t["W2"].data), up(t["gamma"].data), up(t["beta"].data),
                        up(t["gamma"].data), up(t["beta"].data), cfg.world, cfg.batch, cfg.seq,
                        cfg.n_heads, cfg.head_dim, True, cfg.eps)
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    stream = torch.cuda.current_stream()
    stage_keys = ("pre_ln", "attn", "reduce1", "mlp_col", "mlp_row", "reduce2")
    ev = {k: [] for k in stage_keys}
    step = stage_step(cfg, blk, stream, ev)

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"{args.steps} timed steps in {elapsed:.3f} s")
    clock = None
    if not args.no_clock:
        log("clock sampling over ~6 s of steps")
        clock = clock_leg(step, elapsed / args.steps * 1e3)
    sclk = (clock or {}).get("sclk_mhz") or {}
    sclk_ghz = sclk.get("median", 0) / 1e3 if sclk else None
    ceiling = None
    if not args.no_mfma_ceiling:
        log("matrix-core rate calibration")
        ceiling = mfma_ceiling_leg(dev, blk.X, blk.W1)
    ceil_tf = (ceiling or {}).get("tflops")

    def avg_ms(key):  # per launch: the stage's event interval over its launches
        return float(np.mean([s.elapsed_time(e) for s, e in ev[key]])) / LAUNCHES[key]

    fl = rank_flops(cfg)
    step_flops = cfg.world * sum(fl.values())
    value = step_flops * args.steps / elapsed / 1e12
    ms_step = elapsed / args.steps * 1e3

    T, H = cfg.tokens, cfg.hidden
    r1_bytes = reduce_bytes(T, H, cfg.world, "bf16", residual=True, h_out=True, y_out=True)
    r2_bytes = reduce_bytes(T, H, cfg.world, "bf16", residual=True, h_out=True, y_out=False)
    ln_bytes = reduce_bytes(T, H, 0, "bf16", residual=True, h_out=False, y_out=True)
    stages = {}
    for key in ev:
        ms = avg_ms(key)
        entry = {"avg_ms": round(ms, 4), "launches_per_step": LAUNCHES[key]}
        if key == "attn":
            entry["tflops"] = round((fl["qkv"] + fl["attn_core"] + fl["o_proj"]) / ms / 1e9, 1)
        elif key in ("mlp_col", "mlp_row"):
            entry["tflops"] = round(fl[key] / ms / 1e9, 1)
        elif key in ("reduce1", "reduce2", "pre_ln"):
            nbytes = {"reduce1": r1_bytes, "reduce2": r2_bytes, "pre_ln": ln_bytes}[key]
            entry["gbs"] = round(nbytes / ms / 1e6, 1)
            entry["hbm_frac"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)
        stages[key] = entry
    if not args.no_cold:
        log("cold-cache pass over the stages")
        cold = cold_stages(cfg, blk, stream, CacheFlush(dev), max(2, min(args.steps, 5)))
        for key, ms in cold.items():
            e = stages[key]
            e["cold_avg_ms"] = round(ms, 4)
            if "tflops" in e:
                fl_key = (fl["qkv"] + fl["attn_core"] + fl["o_proj"]) if key == "attn" else fl[key]
                e["cold_tflops"] = round(fl_key / ms / 1e9, 1)
            if "gbs" in e:
                nbytes = {"reduce1": r1_bytes, "reduce2": r2_bytes, "pre_ln": ln_bytes}[key]
                e["cold_gbs"] = round(nbytes / ms / 1e6, 1)
                e["cold_hbm_frac"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)

    # Roofline of the MLP's two GEMMs, each one launch shape (8192 x 12288 x 6144 and
    # 8192 x 6144 x 12288, 1236.95 GFLOP): flops per launch over the launch's average duration
    # from the timed steps' events.  `roofline` is the one with more time per step.
    kernels = {"mlp_col": "gemm_bf16_kernel<256,256,EPI_GELU_TANH,LAY_NN> (MLP column GEMM + "
                          "GeLU, 8192x12288x6144, bf16 out)",
               "mlp_row": "gemm_bf16_kernel<256,256,EPI_PARTIAL_F32,LAY_NN> (MLP row GEMM, "
                          "8192x6144x12288, fp32 partial)"}
    rooflines = {}
    for key, name in kernels.items():
        ms = avg_ms(key)
        achieved = fl[key] / (ms * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": name, "achieved": round(achieved, 1),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(key),
             "flops_per_launch": fl[key], "avg_launch_ms": round(ms, 4),
             "time_per_step_ms": round(ms * LAUNCHES[key], 4)}
        if sclk_ghz:
            r["frac_at_measured_sclk"] = round(achieved / (PEAK_BF16_TFLOPS * sclk_ghz / 2.4), 4)
        if ceil_tf:
            r["frac_of_mfma_ceiling"] = round(achieved / ceil_tf, 4)
        rooflines[key] = r
    dominant = max(rooflines, key=lambda k: rooflines[k]["time_per_step_ms"])

    result = {
        "metric": "TFLOP/s per TP-rank layer shard (MLP+attn) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("block_bf16_tp8: Transformer block shard, H=12288, 96 heads x 128, "
                         "FFN 49152, 8 simulated TP ranks computed in turn, batch 4 x seq 2048, "
                         "causal"),
            "global_batch": cfg.batch, "seq_len": cfg.seq, "tp_ranks_simulated": cfg.world,
            "parallelism": "tp8 simulated on 1 GPU",
            "step_gflop": round(step_flops / 1e9, 1),
            "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        },
        "roofline": rooflines[dominant],
        "rooflines": rooflines,
        "clock": clock,
        "mfma_ceiling": ceiling,
        "stages": stages,
        # One simulated rank's layer shard (its attention-head shard and its MLP shard), the
        # unit the metric names: the rank's algorithmic flops over the sum of its stages'
        # per-launch times (the reduces and the pre-LayerNorm are the all-reduce replacement
        # and are left out here; `value` includes them).
        "rank_shard": rank_shard(fl, stages, sclk_ghz),
    }
    if sclk_ghz:
        result["config"]["pct_of_bf16_peak_at_measured_sclk"] = round(
            100 * value / (PEAK_BF16_TFLOPS * sclk_ghz / 2.4), 2)
    # Sequence-parallel epilogue (outside the timed step): rank r's reduce-scatter of the 8
    # partials over its 1024 rows, fused with the residual add and LayerNorm, into its rows of
    # the full buffers (the all-gather).  Same kernel as reduce1, on a row range.
    sp_ev = []
    for it in range(3):  # the 8 ranks back to back, timed as a group
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        for r in range(cfg.world):
            blk.reduce1_scatter(r)
        e_.record(stream)
        if it > 0:
            sp_ev.append((s_, e_))
    torch.cuda.synchronize()
    sp_ms = float(np.mean([s_.elapsed_time(e_) for s_, e_ in sp_ev])) / cfg.world
    sp_bytes = reduce_bytes(T // cfg.world, H, cfg.world, "bf16", residual=True, h_out=True,
                            y_out=True)
    result["sequence_parallel_epilogue"] = {
        "what": "one rank's reduce-scatter (8 fp32 partials, 1024 rows) + residual + LayerNorm",
        "avg_ms_per_rank": round(sp_ms, 4),
        "gbs": round(sp_bytes / sp_ms / 1e6, 1),
        "hbm_frac": round(sp_bytes / sp_ms / 1e6 / PEAK_HBM_GBS, 3),
        "all_ranks_ms": round(sp_ms * cfg.world, 4),
    }
    if not args.no_backward:
        result["mlp_backward"] = mlp_backward_leg(cfg, t, blk, stream)
    if not args.no_workloads:
        log("timing the other workloads")
        result["other_workloads"] = other_workloads_leg(
            dev, flush=None if args.no_cold else CacheFlush(dev), cpu=not args.no_cpu_baseline)
    if not args.no_fold:
        log("timing the block step with folded reduces")
        result["folded_step"] = folded_block_leg(cfg, blk, stream, max(1, min(args.steps, 5)))
    if not args.no_bf16_partials:
        log("timing the block step with bf16 partials")
        result["bf16_partials_step"] = folded_block_leg(cfg, blk, stream,
                                                        max(1, min(args.steps, 5)), "bf16")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(cfg, t, np.hstack(
            [t["Wq"].values(), t["Wk"].values(), t["Wv"].values()]))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
