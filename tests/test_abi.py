"""C-ABI library tests that need no GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from bit_w4a4_quantized_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

OK, NULL, SHAPE, ALIGN, FORMAT, WORKSPACE = 0, -1, -2, -3, -4, -5
P = 4096          # a fake, 16-byte aligned "device" pointer: never dereferenced on these paths
MIS = 4100        # misaligned


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = binding.lib()
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(binding._SIGS), "binding signatures out of sync with the header"


def test_version_and_status_strings():
    assert "gfx950" in binding.version()
    for s in (OK, NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, -6, -7):
        assert binding.status_string(s)
    assert binding.status_string(12345) == "unknown status"


def test_sizes():
    assert binding.code_row_bytes(3072, "int4") == 1536
    assert binding.code_row_bytes(3072, "int8") == 3072
    assert binding.code_row_bytes(3072, "fp4") == 1536
    L = binding.lib()
    assert L.svdq_scale_row_bytes(3072, 0) == 96
    assert L.svdq_scale_row_bytes(3072, 2) == 192
    assert L.svdq_scale_row_bytes(3072, 4) == 96           # MXFP4: one E8M0 byte per 32
    assert L.svdq_code_row_bytes(3072, 4) == 1536
    assert L.svdq_code_row_bytes(100, 0) == 0
    assert L.svdq_code_row_bytes(64, 7) == 0
    # codes + scales + T + Kernel A's partial sums, each 256-byte aligned
    M, K, r = 4608, 3072, 32
    part = binding.quantize_down_workspace_bytes(M, K, r, "int4")
    exp = sum(((b + 255) // 256) * 256 for b in (M * K // 2, M * K // 64 * 2, M * r * 2)) + part
    assert binding.linear_workspace_bytes(M, K, r, "int4") == exp
    assert binding.linear_workspace_bytes(M, 100, r, "int4") == 0
    assert binding.linear_unfused_workspace_bytes(M, 9216, K, r, "int4") == exp + M * 9216 * 2


def test_quantize_down_workspace_sizes():
    # fp32 partial sums of T: a whole number (>= 2) of [M, r] slices when K is sliced
    for M, K, r in [(4608, 3072, 32), (4608, 12288, 32), (4608, 12288, 64), (300, 2048, 16)]:
        b = binding.quantize_down_workspace_bytes(M, K, r, "int4_e2m3")
        assert b % 256 == 0 and b >= 2 * M * r * 4, (M, K, r, b)
        slices = b // (M * r * 4)
        assert slices * M * r * 4 <= b < (slices + 1) * M * r * 4
        assert slices <= K // 64
    assert binding.quantize_down_workspace_bytes(4608, 3072, 0, "int4") == 0     # no branch, no partials
    assert binding.quantize_down_workspace_bytes(16, 128, 16, "int4") == 0       # one slice
    assert binding.quantize_down_workspace_bytes(16, 100, 16, "int4") == 0       # bad shape
    assert binding.quantize_down_workspace_bytes(16, 128, 16, 9) == 0            # bad format


def qd(x=P, l1=P, M=16, K=64, r=16, fmt=0, xq=P, xs=P, t=P, ws=None, ws_bytes=0):
    return binding.lib().svdq_quantize_down(x, l1, M, K, r, fmt, xq, xs, t, ws, ws_bytes, None)


def test_quantize_down_validation():
    assert qd(x=None) == NULL
    assert qd(xq=None) == NULL
    assert qd(l1=None) == NULL
    assert qd(l1=None, t=None, r=0, xq=None) == NULL
    assert qd(K=100) == SHAPE
    assert qd(K=0) == SHAPE
    assert qd(M=-1) == SHAPE
    assert qd(r=8) == SHAPE
    assert qd(r=80) == SHAPE
    assert qd(fmt=5) == FORMAT
    assert qd(x=MIS) == ALIGN
    assert qd(t=MIS) == ALIGN
    assert qd(M=0) == OK            # empty input: nothing enqueued
    assert qd(M=0, r=0, l1=None, t=None) == OK
    assert qd(M=0, x=None, xq=None, xs=None, l1=None, t=None) == OK   # zero-size tensors have NULL data
    assert qd(M=0, K=100) == SHAPE
    # a workspace that is given must be aligned and large enough (checked before any launch)
    M, K = 4608, 3072
    need = binding.quantize_down_workspace_bytes(M, K, 16, "int4")
    assert need > 0
    assert qd(M=M, K=K, ws=P, ws_bytes=need - 256) == WORKSPACE
    assert qd(M=M, K=K, ws=MIS, ws_bytes=need) == ALIGN


def gm(xq=P, xs=P, t=P, wq=P, ws=P, l2=P, bias=P, M=16, N=16, K=64, r=16, fmt=0, y=P):
    return binding.lib().svdq_gemm_w4a4_up(xq, xs, t, wq, ws, l2, bias, M, N, K, r, fmt, y, None)


def test_gemm_validation():
    assert gm(y=None) == NULL
    assert gm(t=None) == NULL
    assert gm(l2=None) == NULL
    assert gm(N=24) == SHAPE
    assert gm(K=32) == SHAPE
    assert gm(fmt=-1) == FORMAT
    assert gm(bias=MIS) == ALIGN
    assert gm(wq=MIS) == ALIGN
    assert gm(M=0) == OK
    assert gm(N=0) == OK


def test_linear_validation():
    L = binding.lib()
    need = L.svdq_linear_workspace_bytes(16, 64, 16, 0)
    f = lambda ws=P, nbytes=need, M=16, N=16, K=64, r=16, fmt=0, x=P, l1=P: L.svdq_linear(
        x, l1, P, P, P, None, M, N, K, r, fmt, ws, nbytes, P, None)
    assert f(nbytes=need - 1) == WORKSPACE
    assert f(ws=None) == NULL
    assert f(ws=MIS) == ALIGN
    assert f(l1=None) == NULL
    assert f(fmt=9) == FORMAT
    assert f(M=0) == OK
    g = lambda nbytes, M=16, N=16: L.svdq_linear_unfused(P, P, P, P, P, None, M, N, 64, 16, 0, P, nbytes, P, None)
    needu = L.svdq_linear_unfused_workspace_bytes(16, 16, 64, 16, 0)
    assert needu > need
    assert g(needu - 1) == WORKSPACE
    assert g(needu, M=0) == OK


def test_weight_gelu_w4a16_validation():
    L = binding.lib()
    assert L.svdq_quantize_weight(None, 16, 64, 0, P, P, None) == NULL
    assert L.svdq_quantize_weight(P, 15, 64, 0, P, P, None) == SHAPE
    assert L.svdq_quantize_weight(P, 16, 64, 5, P, P, None) == FORMAT
    assert L.svdq_quantize_weight(P, 0, 64, 0, P, P, None) == OK
    assert L.svdq_gelu_tanh_smooth(P, P, 4, 12, P, None) == SHAPE
    assert L.svdq_gelu_tanh_smooth(P, None, 4, 16, P, None) == NULL
    assert L.svdq_gelu_tanh_smooth(P, P, 0, 16, P, None) == OK
    assert L.svdq_gemm_w4a16(P, P, P, None, 4, 16, 96, P, None) == SHAPE
    assert L.svdq_gemm_w4a16(P, P, MIS, None, 4, 16, 64, P, None) == ALIGN
    assert L.svdq_gemm_w4a16(P, P, P, None, 0, 16, 64, P, None) == OK


def test_folded_entry_points_validation():
    # the steps folded into the kernels: the factor vectors are required where the entry point
    # names them, and checked for alignment; everything else as for the plain entry points
    L = binding.lib()
    qs = lambda x=P, lam=P, l1=P, M=16, K=64, r=16, fmt=0, xq=P: L.svdq_quantize_down_smooth(
        x, lam, l1, M, K, r, fmt, xq, P, P, None, 0, None)
    assert qs(lam=None) == NULL
    assert qs(lam=MIS) == ALIGN
    assert qs(x=None) == NULL
    assert qs(K=96) == SHAPE
    assert qs(fmt=7) == FORMAT
    assert qs(M=0, lam=None) == OK
    gg = lambda lam=P, M=16, N=16, bias=P, fmt=0: L.svdq_gemm_w4a4_up_gelu_smooth(
        P, P, P, P, P, P, bias, lam, M, N, 64, 16, fmt, P, None)
    assert gg(lam=None) == NULL
    assert gg(lam=MIS) == ALIGN
    assert gg(bias=MIS) == ALIGN
    assert gg(N=24) == SHAPE
    assert gg(N=0, lam=None) == OK
    need = L.svdq_linear_workspace_bytes(16, 64, 16, 0)
    lf = lambda lam_in=None, lam_next=None, nbytes=need, ws=P, M=16: L.svdq_linear_folded(
        P, lam_in, P, P, P, P, None, lam_next, M, 16, 64, 16, 0, ws, nbytes, P, None)
    assert lf(lam_in=MIS) == ALIGN
    assert lf(lam_next=MIS) == ALIGN
    assert lf(nbytes=need - 1) == WORKSPACE
    assert lf(ws=None) == NULL
    assert lf(M=0) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_pack_weight_validation():
    L = binding.lib()
    pk = lambda c=P, s=P, N=16, K=64, fmt=0, wq=P: L.svdq_pack_weight(c, s, N, K, fmt, wq, P, None)
    assert pk(fmt=2) == FORMAT                 # FP4 and MXFP4 codes are not packed from ints
    assert pk(fmt=4) == FORMAT
    assert pk(c=None) == NULL
    assert pk(K=96) == SHAPE
    assert pk(N=24) == SHAPE
    assert pk(wq=MIS) == ALIGN
    assert pk(N=0) == OK


def test_relayout_validation():
    L = binding.lib()
    rl = lambda ci=P, si=P, rows=16, K=64, fmt=3, d=1, co=P, so=P: L.svdq_relayout(ci, si, rows, K, fmt, d, co, so,
                                                                                    None)
    assert rl(ci=None) == NULL
    assert rl(so=None) == NULL
    assert rl(K=96) == SHAPE
    assert rl(K=0) == SHAPE
    assert rl(rows=-1) == SHAPE
    assert rl(d=2) == SHAPE                    # direction is 0 or 1
    assert rl(fmt=5) == FORMAT
    assert rl(co=MIS) == ALIGN
    assert rl(si=MIS) == ALIGN
    assert rl(rows=0, ci=None, si=None, co=None, so=None) == OK



def test_relayout_shapes():
    # exchange layout: row-major codes (K/2 bytes a row, K for INT8) and [rows, K/G] scales
    assert binding.canonical_code_shape(300, 320, "int4_e2m3") == (300, 160)
    assert binding.canonical_code_shape(300, 320, "int8") == (300, 320)
    assert binding.canonical_scale_shape(300, 320, "fp4") == (300, 20)
    assert binding.canonical_scale_shape(300, 320, "mxfp4") == (300, 10)
    assert binding.canonical_scale_shape(300, 320, "int4_e2m3") == (300, 5)
