"""The C-ABI library without a GPU: it loads, exports every function tp_shard.h declares,
and rejects every invalid argument before any HIP call (so these calls launch nothing).

Pointers here are fake, never dereferenced addresses; the module is skipped where a GPU is
visible so that a validation bug can never turn into a launch on a real device."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT, gpu_available

pytestmark = pytest.mark.skipif(gpu_available(), reason="host-only validation tests")

HEADER = os.path.join(ROOT, "include", "tp_shard.h")


@pytest.fixture(scope="module")
def tp():
    from megatron_tensor_transformer_linear_amd import _build
    if not os.path.exists(_build.LIB_PATH):
        _build.build_library()
    from megatron_tensor_transformer_linear_amd import tp as mod
    return mod


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tp_col_linear_gelu", "tp_row_linear_partial", "tp_attn_head_shard",
              "tp_partial_reduce_residual_ln", "tp_attn_workspace_bytes", "tp_status_string",
              "tp_partial_reduce_scatter_residual_ln", "tp_col_linear_gelu_save",
              "tp_row_linear_backward", "tp_col_linear_backward",
              "tp_col_linear_backward_bf16"):
        assert n in names


def test_library_exports_every_declared_symbol(tp):
    lib = ctypes.CDLL(tp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (tp_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    assert set(tp.EXPORTED) == set(declared_functions())


def test_calibration_library_loads_and_rejects_bad_arguments(tp):
    """The bench's matrix-core rate calibration library is built beside the main one; bad
    arguments are refused before any launch."""
    from megatron_tensor_transformer_linear_amd import _build
    assert os.path.exists(_build.CALIB_LIB_PATH)
    lib = ctypes.CDLL(_build.CALIB_LIB_PATH)
    lib.tp_calib_mfma_loop.restype = ctypes.c_int
    lib.tp_calib_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.tp_calib_mfma_flops.restype = ctypes.c_double
    lib.tp_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    p = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is refused first
    assert lib.tp_calib_mfma_loop(None, p, 4096, p, 512, 10, None) == -1
    assert lib.tp_calib_mfma_loop(p, p, 4096, None, 512, 10, None) == -1
    assert lib.tp_calib_mfma_loop(p, p, 4096, p, 0, 10, None) == -1
    assert lib.tp_calib_mfma_loop(p, p, 4096, p, 512, 0, None) == -1
    assert lib.tp_calib_mfma_loop(p, p, 4100, p, 512, 10, None) == -1
    assert lib.tp_calib_mfma_loop(p, p, 0, p, 512, 10, None) == -1
    assert lib.tp_calib_mfma_loop(ctypes.c_void_p(0x1008), p, 4096, p, 512, 10, None) == -1
    # 512 workgroups x 4 waves x 10 rounds x 16 MFMAs x 32768 flops
    assert lib.tp_calib_mfma_flops(512, 10) == 512 * 4 * 10 * 16 * 32768


def test_status_strings(tp):
    for code in range(0, -10, -1):
        s = tp.tp_status_string(code)
        assert s.startswith("TP_OK" if code == 0 else "TP_ERR_")
    assert tp.tp_status_string(-100) == "unknown tp_status"


P = 0x10000  # fake, 256-byte aligned, never dereferenced


def col(tp, **kw):
    a = dict(X=P, W=P, Y=P, ldy=512, seq=64, H=256, N=1024, rank=0, world=2,
             act=tp.TP_ACT_GELU_TANH, dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_col_linear_gelu(a["X"], a["W"], a["Y"], a["ldy"], a["seq"], a["H"], a["N"],
                                     a["rank"], a["world"], a["act"], a["dtype"], a["stream"])


def row(tp, **kw):
    a = dict(X=P, ldx=1024, W=P, Z=P, seq=64, K=1024, N=256, rank=1, world=2, dtype=tp.TP_BF16,
             stream=None)
    a.update(kw)
    return tp.lib.tp_row_linear_partial(a["X"], a["ldx"], a["W"], a["Z"], a["seq"], a["K"], a["N"],
                                        a["rank"], a["world"], a["dtype"], a["stream"])


def attn(tp, **kw):
    a = dict(Xn=P, Wqkv=P, Wo=P, Z=P, batch=2, seq=64, H=1024, nh=8, d=128, rank=0, world=4,
             causal=1, dtype=tp.TP_BF16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return tp.lib.tp_attn_head_shard(a["Xn"], a["Wqkv"], a["Wo"], a["Z"], a["batch"], a["seq"],
                                     a["H"], a["nh"], a["d"], a["rank"], a["world"], a["causal"],
                                     a["dtype"], a["ws"], a["wsb"], a["stream"])


def attnn(tp, **kw):
    a = dict(Xn=P, Wqkv=P, Wo=P, Z=P, batch=2, seq=64, H=1024, nh=8, d=128, rank=0, world=4,
             causal=1, dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_attn_head_shard_noalloc(a["Xn"], a["Wqkv"], a["Wo"], a["Z"], a["batch"],
                                             a["seq"], a["H"], a["nh"], a["d"], a["rank"],
                                             a["world"], a["causal"], a["dtype"], a["stream"])


def rowf(tp, **kw):
    a = dict(X=P, ldx=1024, W=P, Z=P, seq=64, K=1024, N=256, rank=1, world=2, acc=1,
             dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_row_linear_fold(a["X"], a["ldx"], a["W"], a["Z"], a["seq"], a["K"], a["N"],
                                     a["rank"], a["world"], a["acc"], a["dtype"], a["stream"])


def attnf(tp, **kw):
    a = dict(Xn=P, Wqkv=P, Wo=P, Z=P, batch=2, seq=64, H=1024, nh=8, d=128, rank=1, world=4,
             causal=1, acc=1, dtype=tp.TP_BF16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return tp.lib.tp_attn_head_shard_fold(a["Xn"], a["Wqkv"], a["Wo"], a["Z"], a["batch"],
                                          a["seq"], a["H"], a["nh"], a["d"], a["rank"],
                                          a["world"], a["causal"], a["acc"], a["dtype"], a["ws"],
                                          a["wsb"], a["stream"])


def red(tp, **kw):
    a = dict(parts=P, n=4, stride=64 * 256, res=P, g=P, b=P, eps=1e-5, h=P, y=P, rows=64, H=256,
             dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_partial_reduce_residual_ln(a["parts"], a["n"], a["stride"], a["res"], a["g"],
                                                a["b"], a["eps"], a["h"], a["y"], a["rows"],
                                                a["H"], a["dtype"], a["stream"])


def rs(tp, **kw):
    a = dict(parts=P, n=4, stride=64 * 256, res=P, g=P, b=P, eps=1e-5, h=P, y=P, rows=64, H=256,
             rank=1, world=4, dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_partial_reduce_scatter_residual_ln(
        a["parts"], a["n"], a["stride"], a["res"], a["g"], a["b"], a["eps"], a["h"], a["y"],
        a["rows"], a["H"], a["rank"], a["world"], a["dtype"], a["stream"])


def cols(tp, **kw):
    a = dict(X=P, W=P, Y=P, ldy=512, U=P, ldu=512, seq=64, H=256, N=1024, rank=1, world=2,
             dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_col_linear_gelu_save(a["X"], a["W"], a["Y"], a["ldy"], a["U"], a["ldu"],
                                          a["seq"], a["H"], a["N"], a["rank"], a["world"],
                                          a["dtype"], a["stream"])


def rowb(tp, **kw):
    a = dict(dZ=P, W=P, Y=P, ldy=512, U=P, ldu=512, dY=P, ld_dy=512, dW=P, ld_dw=256, seq=64,
             K=1024, N=256, rank=1, world=2, act=tp.TP_ACT_GELU_TANH, acc=0, dtype=tp.TP_BF16,
             stream=None)
    a.update(kw)
    return tp.lib.tp_row_linear_backward(a["dZ"], a["W"], a["Y"], a["ldy"], a["U"], a["ldu"],
                                         a["dY"], a["ld_dy"], a["dW"], a["ld_dw"], a["seq"],
                                         a["K"], a["N"], a["rank"], a["world"], a["act"], a["acc"],
                                         a["dtype"], a["stream"])


def colb(tp, **kw):
    a = dict(X=P, W=P, dU=P, ldu=512, dX=P, dW=P, ld_dw=512, seq=64, H=256, N=1024, rank=0,
             world=2, acc=1, dtype=tp.TP_BF16, stream=None)
    a.update(kw)
    return tp.lib.tp_col_linear_backward(a["X"], a["W"], a["dU"], a["ldu"], a["dX"], a["dW"],
                                         a["ld_dw"], a["seq"], a["H"], a["N"], a["rank"],
                                         a["world"], a["acc"], a["dtype"], a["stream"])


def colbh(tp, **kw):
    a = dict(X=P, W=P, dU=P, ldu=512, dX=P, dW=P, ld_dw=512, seq=64, H=256, N=1024, rank=0,
             world=2, acc=1, stream=None)
    a.update(kw)
    return tp.lib.tp_col_linear_backward_bf16(a["X"], a["W"], a["dU"], a["ldu"], a["dX"], a["dW"],
                                              a["ld_dw"], a["seq"], a["H"], a["N"], a["rank"],
                                              a["world"], a["acc"], a["stream"])


def rowh(tp, **kw):
    a = dict(X=P, ldx=1024, W=P, Z=P, seq=64, K=1024, N=256, rank=1, world=2, stream=None)
    a.update(kw)
    return tp.lib.tp_row_linear_partial_bf16(a["X"], a["ldx"], a["W"], a["Z"], a["seq"], a["K"],
                                             a["N"], a["rank"], a["world"], a["stream"])


def attnh(tp, **kw):
    a = dict(Xn=P, Wqkv=P, Wo=P, Z=P, batch=2, seq=64, H=1024, nh=8, d=128, rank=0, world=4,
             causal=1, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return tp.lib.tp_attn_head_shard_bf16(a["Xn"], a["Wqkv"], a["Wo"], a["Z"], a["batch"],
                                          a["seq"], a["H"], a["nh"], a["d"], a["rank"],
                                          a["world"], a["causal"], a["ws"], a["wsb"], a["stream"])


def redh(tp, **kw):
    a = dict(parts=P, n=4, stride=64 * 256, res=P, g=P, b=P, eps=1e-5, h=P, y=P, rows=64, H=256,
             stream=None)
    a.update(kw)
    return tp.lib.tp_partial_reduce_residual_ln_bf16(a["parts"], a["n"], a["stride"], a["res"],
                                                     a["g"], a["b"], a["eps"], a["h"], a["y"],
                                                     a["rows"], a["H"], a["stream"])


def rsh(tp, **kw):
    a = dict(parts=P, n=4, stride=64 * 256, res=P, g=P, b=P, eps=1e-5, h=P, y=P, rows=64, H=256,
             rank=1, world=4, stream=None)
    a.update(kw)
    return tp.lib.tp_partial_reduce_scatter_residual_ln_bf16(
        a["parts"], a["n"], a["stride"], a["res"], a["g"], a["b"], a["eps"], a["h"], a["y"],
        a["rows"], a["H"], a["rank"], a["world"], a["stream"])


CASES = [
    # column-parallel linear
    ("col null X", col, dict(X=None), "TP_ERR_NULL"),
    ("col null W", col, dict(W=None), "TP_ERR_NULL"),
    ("col null Y", col, dict(Y=None), "TP_ERR_NULL"),
    ("col bad dtype", col, dict(dtype=7), "TP_ERR_DTYPE"),
    ("col bad act", col, dict(act=3), "TP_ERR_DTYPE"),
    ("col world 0", col, dict(world=0), "TP_ERR_RANK"),
    ("col rank = world", col, dict(rank=2), "TP_ERR_RANK"),
    ("col rank < 0", col, dict(rank=-1), "TP_ERR_RANK"),
    ("col seq 0", col, dict(seq=0), "TP_ERR_SHAPE"),
    ("col H 0", col, dict(H=0), "TP_ERR_SHAPE"),
    ("col N negative", col, dict(N=-8), "TP_ERR_SHAPE"),
    ("col N % world", col, dict(N=1024, world=3, rank=0, ldy=1024), "TP_ERR_DIVISIBLE"),
    ("col ldy < N/world", col, dict(ldy=504), "TP_ERR_SHAPE"),
    ("col misaligned X", col, dict(X=P + 2), "TP_ERR_ALIGN"),
    ("col misaligned Y", col, dict(Y=P + 8), "TP_ERR_ALIGN"),
    ("col H % 8", col, dict(H=252), "TP_ERR_ALIGN"),
    ("col N/world % 8", col, dict(N=1028, world=2, ldy=1028), "TP_ERR_ALIGN"),
    ("col ldy % 8", col, dict(ldy=516), "TP_ERR_ALIGN"),
    ("col H beyond 2^21", col, dict(H=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("col N beyond 2^23", col, dict(N=(1 << 23) + 16, ldy=(1 << 22) + 8), "TP_ERR_SHAPE"),
    # row-parallel partial
    ("row null X", row, dict(X=None), "TP_ERR_NULL"),
    ("row null Z", row, dict(Z=None), "TP_ERR_NULL"),
    ("row bad dtype", row, dict(dtype=2), "TP_ERR_DTYPE"),
    ("row rank > world", row, dict(rank=5), "TP_ERR_RANK"),
    ("row K 0", row, dict(K=0), "TP_ERR_SHAPE"),
    ("row ldx < K/world", row, dict(ldx=504), "TP_ERR_SHAPE"),
    ("row K % world", row, dict(K=1024, world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("row K/world % 8", row, dict(K=1032, ldx=1032, world=2), "TP_ERR_ALIGN"),
    ("row misaligned W", row, dict(W=P + 4), "TP_ERR_ALIGN"),
    ("row ldx % 8", row, dict(ldx=1028), "TP_ERR_ALIGN"),
    ("row ldx beyond 2^21", row, dict(ldx=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("row N beyond 2^23", row, dict(N=(1 << 23) + 8), "TP_ERR_SHAPE"),
    # row-parallel linear folded into the running sum
    ("fold null X", rowf, dict(X=None), "TP_ERR_NULL"),
    ("fold null W", rowf, dict(W=None), "TP_ERR_NULL"),
    ("fold null Z", rowf, dict(Z=None), "TP_ERR_NULL"),
    ("fold bad dtype", rowf, dict(dtype=2), "TP_ERR_DTYPE"),
    ("fold rank = world", rowf, dict(rank=2), "TP_ERR_RANK"),
    ("fold world 0", rowf, dict(world=0, rank=0), "TP_ERR_RANK"),
    ("fold seq 0", rowf, dict(seq=0), "TP_ERR_SHAPE"),
    ("fold ldx < K/world", rowf, dict(ldx=504), "TP_ERR_SHAPE"),
    ("fold K % world", rowf, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("fold misaligned Z", rowf, dict(Z=P + 4), "TP_ERR_ALIGN"),
    ("fold N % 8", rowf, dict(N=252), "TP_ERR_ALIGN"),
    ("fold ldx beyond 2^21", rowf, dict(ldx=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("fold first rank null Z", rowf, dict(Z=None, acc=0, rank=0), "TP_ERR_NULL"),
    # row-parallel partial in bf16
    ("row bf16 null X", rowh, dict(X=None), "TP_ERR_NULL"),
    ("row bf16 null Z", rowh, dict(Z=None), "TP_ERR_NULL"),
    ("row bf16 rank = world", rowh, dict(rank=2), "TP_ERR_RANK"),
    ("row bf16 ldx < K/world", rowh, dict(ldx=504), "TP_ERR_SHAPE"),
    ("row bf16 K % world", rowh, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("row bf16 misaligned Z", rowh, dict(Z=P + 8), "TP_ERR_ALIGN"),
    ("row bf16 N % 8", rowh, dict(N=252), "TP_ERR_ALIGN"),
    # attention-head shard with a bf16 partial
    ("attn bf16 null Z", attnh, dict(Z=None), "TP_ERR_NULL"),
    ("attn bf16 bad rank", attnh, dict(rank=4), "TP_ERR_RANK"),
    ("attn bf16 H != heads*d", attnh, dict(H=1000), "TP_ERR_SHAPE"),
    ("attn bf16 heads % world", attnh, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("attn bf16 small workspace", attnh, dict(wsb=1000), "TP_ERR_WORKSPACE"),
    ("attn bf16 misaligned Z", attnh, dict(Z=P + 8), "TP_ERR_ALIGN"),
    # reduce + residual + LN over bf16 partials
    ("reduce bf16 negative parts", redh, dict(n=-1), "TP_ERR_SHAPE"),
    ("reduce bf16 null parts", redh, dict(parts=None), "TP_ERR_NULL"),
    ("reduce bf16 nothing to read", redh, dict(n=0, parts=None, res=None), "TP_ERR_NULL"),
    ("reduce bf16 gamma without y", redh, dict(y=None), "TP_ERR_NULL"),
    ("reduce bf16 rows 0", redh, dict(rows=0), "TP_ERR_SHAPE"),
    ("reduce bf16 NaN eps", redh, dict(eps=float("nan")), "TP_ERR_SHAPE"),
    ("reduce bf16 stride too small", redh, dict(stride=64 * 256 - 8), "TP_ERR_SHAPE"),
    ("reduce bf16 stride % 8", redh, dict(stride=64 * 256 + 4), "TP_ERR_ALIGN"),
    ("reduce bf16 H % 8", redh, dict(H=252, stride=64 * 252), "TP_ERR_ALIGN"),
    ("reduce bf16 misaligned parts", redh, dict(parts=P + 8), "TP_ERR_ALIGN"),
    # reduce-scatter over bf16 partials
    ("scatter bf16 rows % world", rsh, dict(rows=66, stride=66 * 256), "TP_ERR_DIVISIBLE"),
    ("scatter bf16 rank = world", rsh, dict(rank=4), "TP_ERR_RANK"),
    ("scatter bf16 null parts", rsh, dict(parts=None), "TP_ERR_NULL"),
    ("scatter bf16 gamma without y", rsh, dict(y=None), "TP_ERR_NULL"),
    ("scatter bf16 stride too small", rsh, dict(stride=64 * 256 - 8), "TP_ERR_SHAPE"),
    ("scatter bf16 stride % 8", rsh, dict(stride=64 * 256 + 4), "TP_ERR_ALIGN"),
    ("scatter bf16 misaligned h", rsh, dict(h=P + 4), "TP_ERR_ALIGN"),
    # attention-head shard
    ("attn null Wo", attn, dict(Wo=None), "TP_ERR_NULL"),
    ("attn f32", attn, dict(dtype=0), "TP_ERR_DTYPE"),
    ("attn bad rank", attn, dict(rank=4), "TP_ERR_RANK"),
    ("attn H != heads*d", attn, dict(H=1000), "TP_ERR_SHAPE"),
    ("attn head_dim 64", attn, dict(d=64, nh=16), "TP_ERR_SHAPE"),
    ("attn seq 0", attn, dict(seq=0), "TP_ERR_SHAPE"),
    ("attn H beyond 2^21", attn, dict(H=(1 << 21) + 128 * 4, nh=(1 << 14) + 4), "TP_ERR_SHAPE"),
    ("attn heads % world", attn, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("attn no workspace", attn, dict(ws=None), "TP_ERR_WORKSPACE"),
    ("attn small workspace", attn, dict(wsb=1000), "TP_ERR_WORKSPACE"),
    ("attn misaligned workspace", attn, dict(ws=P + 16), "TP_ERR_ALIGN"),
    ("attn misaligned Xn", attn, dict(Xn=P + 2), "TP_ERR_ALIGN"),
    # attention-head shard folded into the running sum
    ("attn fold null Z", attnf, dict(Z=None), "TP_ERR_NULL"),
    ("attn fold null Xn", attnf, dict(Xn=None), "TP_ERR_NULL"),
    ("attn fold f32", attnf, dict(dtype=0), "TP_ERR_DTYPE"),
    ("attn fold rank = world", attnf, dict(rank=4), "TP_ERR_RANK"),
    ("attn fold head_dim 64", attnf, dict(d=64, nh=16), "TP_ERR_SHAPE"),
    ("attn fold heads % world", attnf, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("attn fold small workspace", attnf, dict(wsb=1000), "TP_ERR_WORKSPACE"),
    ("attn fold misaligned Z", attnf, dict(Z=P + 8), "TP_ERR_ALIGN"),
    # attention-head shard on the library's static scratch (no workspace argument)
    ("attn noalloc null Xn", attnn, dict(Xn=None), "TP_ERR_NULL"),
    ("attn noalloc null Z", attnn, dict(Z=None), "TP_ERR_NULL"),
    ("attn noalloc f32", attnn, dict(dtype=0), "TP_ERR_DTYPE"),
    ("attn noalloc bad rank", attnn, dict(rank=-1), "TP_ERR_RANK"),
    ("attn noalloc H != heads*d", attnn, dict(H=1000), "TP_ERR_SHAPE"),
    ("attn noalloc heads % world", attnn, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("attn noalloc misaligned Wqkv", attnn, dict(Wqkv=P + 8), "TP_ERR_ALIGN"),
    # 8 x 4096 tokens, 12 heads per rank: QKV_r alone is 302 MB, beyond the 160 MiB scratch
    ("attn noalloc beyond the scratch", attnn,
     dict(batch=8, seq=4096, H=12288, nh=96, world=8), "TP_ERR_SCRATCH"),
    # reduce + residual + LN
    ("reduce bad dtype", red, dict(dtype=9), "TP_ERR_DTYPE"),
    ("reduce negative parts", red, dict(n=-1), "TP_ERR_SHAPE"),
    ("reduce null parts", red, dict(parts=None), "TP_ERR_NULL"),
    ("reduce nothing to read", red, dict(n=0, parts=None, res=None), "TP_ERR_NULL"),
    ("reduce gamma without y", red, dict(y=None), "TP_ERR_NULL"),
    ("reduce no output", red, dict(g=None, h=None), "TP_ERR_NULL"),
    ("reduce rows 0", red, dict(rows=0), "TP_ERR_SHAPE"),
    ("reduce H too large", red, dict(H=65544, stride=64 * 65544), "TP_ERR_SHAPE"),
    ("reduce negative eps", red, dict(eps=-1.0), "TP_ERR_SHAPE"),
    ("reduce NaN eps", red, dict(eps=float("nan")), "TP_ERR_SHAPE"),
    ("reduce stride too small", red, dict(stride=64 * 256 - 4), "TP_ERR_SHAPE"),
    ("reduce H % 8", red, dict(H=252, stride=64 * 252), "TP_ERR_ALIGN"),
    ("reduce stride % 4", red, dict(stride=64 * 256 + 2), "TP_ERR_ALIGN"),
    ("reduce misaligned residual", red, dict(res=P + 8), "TP_ERR_ALIGN"),
    ("reduce misaligned y", red, dict(y=P + 2), "TP_ERR_ALIGN"),
    # sequence-parallel reduce-scatter + residual + LN
    ("scatter rows % world", rs, dict(rows=66, stride=66 * 256), "TP_ERR_DIVISIBLE"),
    ("scatter rank = world", rs, dict(rank=4), "TP_ERR_RANK"),
    ("scatter world 0", rs, dict(world=0), "TP_ERR_RANK"),
    ("scatter bad dtype", rs, dict(dtype=3), "TP_ERR_DTYPE"),
    ("scatter null parts", rs, dict(parts=None), "TP_ERR_NULL"),
    ("scatter gamma without y", rs, dict(y=None), "TP_ERR_NULL"),
    ("scatter stride too small", rs, dict(stride=64 * 256 - 8), "TP_ERR_SHAPE"),
    ("scatter H % 8", rs, dict(H=260, stride=64 * 260), "TP_ERR_ALIGN"),
    ("scatter misaligned h", rs, dict(h=P + 4), "TP_ERR_ALIGN"),
    # column-parallel linear keeping the pre-activation
    ("save null U", cols, dict(U=None), "TP_ERR_NULL"),
    ("save null Y", cols, dict(Y=None), "TP_ERR_NULL"),
    ("save f32", cols, dict(dtype=0), "TP_ERR_DTYPE"),
    ("save rank = world", cols, dict(rank=2), "TP_ERR_RANK"),
    ("save ldu < N/world", cols, dict(ldu=504), "TP_ERR_SHAPE"),
    ("save N % world", cols, dict(world=3, rank=0, ldy=1024, ldu=1024), "TP_ERR_DIVISIBLE"),
    ("save ldu % 8", cols, dict(ldu=516), "TP_ERR_ALIGN"),
    ("save misaligned U", cols, dict(U=P + 8), "TP_ERR_ALIGN"),
    # row-parallel backward
    ("rowb null dZ", rowb, dict(dZ=None), "TP_ERR_NULL"),
    ("rowb null W", rowb, dict(W=None), "TP_ERR_NULL"),
    ("rowb no output", rowb, dict(dY=None, dW=None), "TP_ERR_NULL"),
    ("rowb dW without Y", rowb, dict(Y=None), "TP_ERR_NULL"),
    ("rowb gelu without U", rowb, dict(U=None), "TP_ERR_NULL"),
    ("rowb f32", rowb, dict(dtype=0), "TP_ERR_DTYPE"),
    ("rowb bad act", rowb, dict(act=2), "TP_ERR_DTYPE"),
    ("rowb rank < 0", rowb, dict(rank=-1), "TP_ERR_RANK"),
    ("rowb seq 0", rowb, dict(seq=0), "TP_ERR_SHAPE"),
    ("rowb seq beyond 2^30", rowb, dict(seq=(1 << 30) + 8), "TP_ERR_SHAPE"),
    ("rowb K % world", rowb, dict(world=3, rank=0), "TP_ERR_DIVISIBLE"),
    ("rowb ld_dy < K/world", rowb, dict(ld_dy=504), "TP_ERR_SHAPE"),
    ("rowb ldu < K/world", rowb, dict(ldu=504), "TP_ERR_SHAPE"),
    ("rowb ldy < K/world", rowb, dict(ldy=504), "TP_ERR_SHAPE"),
    ("rowb ld_dw < N", rowb, dict(ld_dw=248), "TP_ERR_SHAPE"),
    ("rowb N beyond 2^21", rowb, dict(N=(1 << 21) + 8, ld_dw=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("rowb ldy beyond 2^21", rowb, dict(ldy=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("rowb misaligned dW", rowb, dict(dW=P + 4), "TP_ERR_ALIGN"),
    ("rowb misaligned U", rowb, dict(U=P + 2), "TP_ERR_ALIGN"),
    ("rowb K/world % 8", rowb, dict(K=1032, ldy=520, ldu=520, ld_dy=520), "TP_ERR_ALIGN"),
    ("rowb ld_dw % 8", rowb, dict(ld_dw=260), "TP_ERR_ALIGN"),
    # column-parallel backward
    ("colb null X", colb, dict(X=None), "TP_ERR_NULL"),
    ("colb null dU", colb, dict(dU=None), "TP_ERR_NULL"),
    ("colb no output", colb, dict(dX=None, dW=None), "TP_ERR_NULL"),
    ("colb f32", colb, dict(dtype=0), "TP_ERR_DTYPE"),
    ("colb world 0", colb, dict(world=0), "TP_ERR_RANK"),
    ("colb H 0", colb, dict(H=0), "TP_ERR_SHAPE"),
    ("colb N % world", colb, dict(world=3), "TP_ERR_DIVISIBLE"),
    ("colb ldu < N/world", colb, dict(ldu=504), "TP_ERR_SHAPE"),
    ("colb ld_dw < N/world", colb, dict(ld_dw=504), "TP_ERR_SHAPE"),
    ("colb H beyond 2^21", colb, dict(H=(1 << 21) + 8), "TP_ERR_SHAPE"),
    ("colb N beyond 2^21", colb, dict(N=(1 << 21) + 16, ldu=(1 << 20) + 8, ld_dw=(1 << 20) + 8),
     "TP_ERR_SHAPE"),
    ("colb misaligned dX", colb, dict(dX=P + 8), "TP_ERR_ALIGN"),
    ("colb ldu % 8", colb, dict(ldu=516), "TP_ERR_ALIGN"),
    # column-parallel linear backward, bf16 input-gradient partial
    ("colb bf16 null W", colbh, dict(W=None), "TP_ERR_NULL"),
    ("colb bf16 no output", colbh, dict(dX=None, dW=None), "TP_ERR_NULL"),
    ("colb bf16 rank = world", colbh, dict(rank=2), "TP_ERR_RANK"),
    ("colb bf16 seq 0", colbh, dict(seq=0), "TP_ERR_SHAPE"),
    ("colb bf16 N % world", colbh, dict(world=3), "TP_ERR_DIVISIBLE"),
    ("colb bf16 ld_dw < N/world", colbh, dict(ld_dw=504), "TP_ERR_SHAPE"),
    ("colb bf16 misaligned dX", colbh, dict(dX=P + 8), "TP_ERR_ALIGN"),
    ("colb bf16 H % 8", colbh, dict(H=252), "TP_ERR_ALIGN"),
]


@pytest.mark.parametrize("name,fn,kw,expect", CASES, ids=[c[0] for c in CASES])
def test_validation_rejects_before_launch(tp, name, fn, kw, expect):
    assert fn(tp, **kw) == getattr(tp, expect)


def test_workspace_bytes(tp):
    T, nb = 2 * 64, (8 // 4) * 128
    expect = (T * 3 * nb * 2 + T * nb * 2 + 255) // 256 * 256
    assert tp.tp_attn_workspace_bytes(2, 64, 1024, 8, 128, 4, tp.TP_BF16) == expect
    assert tp.tp_attn_workspace_bytes(2, 64, 1024, 8, 128, 3, tp.TP_BF16) == 0
    assert tp.tp_attn_workspace_bytes(2, 64, 1024, 8, 128, 4, tp.TP_F32) == 0
    assert tp.tp_attn_workspace_bytes(2, 64, 1000, 8, 128, 4, tp.TP_BF16) == 0


def test_workspace_bytes_split_strip(tp):
    """The block's attention shard (8192 tokens, 12 heads per rank): its QKV projection's
    launch plan on 256 compute units (the count assumed when no device can be queried) has a
    512-wide strip, whose split contraction adds 4 fp32 partials of 8192 x 512 to the workspace."""
    T, nb = 4 * 2048, (96 // 8) * 128
    plain = (T * 3 * nb * 2 + T * nb * 2 + 255) // 256 * 256
    assert tp.tp_attn_workspace_bytes(4, 2048, 12288, 96, 128, 8, tp.TP_BF16) == plain + 4 * T * 512 * 4


def test_scratch_limit_fits_the_block_workload(tp):
    """The static scratch holds the workspace of one rank of the largest workload (8192
    tokens, 12 heads of 128 per rank, H = 12288) on 256 compute units, exactly; twice the
    tokens do not fit."""
    need = tp.tp_attn_workspace_bytes(4, 2048, 12288, 96, 128, 8, tp.TP_BF16)
    assert need == tp.TP_ATTN_SCRATCH_BYTES
    assert tp.tp_attn_workspace_bytes(8, 2048, 12288, 96, 128, 8, tp.TP_BF16) > \
        tp.TP_ATTN_SCRATCH_BYTES
    assert attnn(tp, batch=8, seq=2048, H=12288, nh=96, world=8) == tp.TP_ERR_SCRATCH


def test_header_scratch_size_matches_binding(tp):
    src = open(HEADER).read()
    m = re.search(r"#define TP_ATTN_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tp.TP_ATTN_SCRATCH_BYTES


def test_python_wrapper_raises(tp):
    with pytest.raises(tp.TPError) as e:
        tp.tp_col_linear_gelu(P, P, P, 512, 64, 256, 1024, 2, 2, 1, tp.TP_BF16, stream=0)
    assert e.value.status == tp.TP_ERR_RANK
