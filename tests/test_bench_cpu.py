"""The measurement script's contract, without a GPU: one GPU only, and the HBM-traffic
figure tied to the kernel sources it was measured on."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 exits with status 2 and says why, before touching any device."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The traffic figure is reported only while the GEMM sources hash to the digest stored
    beside it; a summary for other sources yields null."""
    src = open(bench.TRAFFIC_FILE).read()
    kv = dict(l.split(": ", 1) for l in src.splitlines() if ": " in l and
              l.split(": ", 1)[0] in ("kernel_sources", "kernel_sources_sha256"))
    h = hashlib.sha256()
    for f in kv["kernel_sources"].split():
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() == kv["kernel_sources_sha256"].strip():
        for role in ("mlp_col", "mlp_row"):
            assert isinstance(bench.measured_traffic(role), int)
    assert bench.measured_traffic("no_such_role") is None
    stale = tmp_path / "traffic.md"
    stale.write_text(src.replace(kv["kernel_sources_sha256"].strip(), "0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("mlp_row") is None
