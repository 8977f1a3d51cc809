"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/gemm.h declares, and rejects invalid arguments on the
host before touching a device."""
import ctypes
import os
import re

import pytest
import torch

import dense_gemm_engineering_amd.binding as dge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = ""
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            with open(os.path.join(ROOT, "include", h)) as f:
                src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+([a-z_0-9]+)\s*\(", src,
                       flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    assert sorted(dge.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    L = dge.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    for s in range(7):
        assert dge.gemm_status_string(s).startswith(dge.STATUS_NAMES[s])
    assert "unknown" in dge.gemm_status_string(99)


def _call(L, **kw):
    a = dict(M=4, N=4, K=4, alpha=1.0, A=8, lda=4, B=4096, ldb=4, trans_b=0, beta=0.0, C=65536,
             ldc=4, c_type=1, epi=0, bias=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.gemm_f16(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"], a["ldb"],
                      a["trans_b"], a["beta"], a["C"], a["ldc"], a["c_type"], a["epi"], a["bias"],
                      a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("bad", [dict(M=-1), dict(K=-2), dict(lda=3), dict(ldb=3), dict(ldc=3),
                                 dict(trans_b=2), dict(c_type=7), dict(epi=3),
                                 dict(epi=1, bias=None), dict(C=None), dict(A=None),
                                 dict(alpha=float("nan")), dict(C=8),  # C overlaps A
                                 dict(trans_b=1, ldb=3), dict(M=1 << 31)])
def test_invalid_arguments_rejected_on_host(bad):
    assert _call(dge.lib(), **bad) == 1


def test_empty_problem_is_ok_without_device():
    assert _call(dge.lib(), M=0) == 0
    assert _call(dge.lib(), N=0, C=None) in (0, 1)


def test_fp32_requires_fp32_output():
    L = dge.lib()
    st = L.gemm_f32(4, 4, 4, 1.0, 8, 4, 4096, 4, 0, 0.0, 65536, 4, 1, 0, None, None, 0, None)
    assert st == 1


def test_dequant_validation():
    L = dge.lib()
    assert L.dequant_q4_f16(2, 4096, 4, 16, 16, None) == 1   # cols not a multiple of 32
    assert L.dequant_q4_f16(3, 4096, 4, 32, 32, None) == 1   # odd q address
    assert L.dequant_q4_f16(2, 4096, 4, 32, 31, None) == 1   # ldo < cols
    assert L.dequant_q4_f16(2, 4096, 0, 32, 32, None) == 0   # empty


def test_prefill_validation():
    L = dge.lib()
    # K not a multiple of 32
    assert L.prefill_q4_f16(4, 4, 40, 8, 40, 4096, 1 << 20, 1 << 24, 4, 1, 0, None, None, 0,
                            None) == 1


def test_fused_q4_validation():
    L = dge.lib()
    # K not a multiple of 32; odd q address; bad tuning algo
    assert L.gemm_q4_f16(4, 4, 40, 8, 40, 4096, 1 << 24, 4, 1, 0, None, None, 0, None,
                         None) == 1
    assert L.gemm_q4_f16(4, 4, 64, 8, 64, 4097, 1 << 24, 4, 1, 0, None, None, 0, None,
                         None) == 1
    t = dge.Tuning(dge.ALGO["naive"], 0, 0)
    assert L.gemm_q4_f16(4, 4, 64, 8, 64, 4096, 1 << 24, 4, 1, 0, None, None, 0,
                         ctypes.byref(t), None) == 1
    # empty problem
    assert L.gemm_q4_f16(0, 4, 64, 8, 64, 4096, 1 << 24, 4, 1, 0, None, None, 0, None,
                         None) == 0


def test_kquant_validation():
    L = dge.lib()
    # unknown format; cols not a multiple of 256; ldo < cols; odd out address
    assert L.dequant_f16(4, 4096, 1 << 24, 4, 256, 256, None) == 1
    assert L.dequant_f16(-1, 4096, 1 << 24, 4, 256, 256, None) == 1
    assert L.dequant_f16(1, 4096, 1 << 24, 4, 224, 224, None) == 1
    assert L.dequant_f16(2, 4096, 1 << 24, 4, 256, 255, None) == 1
    assert L.dequant_f16(2, 4096, (1 << 24) + 1, 4, 256, 256, None) == 1
    # q overlapping out
    assert L.dequant_f16(2, 1 << 24, (1 << 24) + 64, 4, 256, 256, None) == 1
    # q4_0 keeps its own rules (cols % 32, q 2-byte aligned)
    assert L.dequant_f16(0, 4097, 1 << 24, 4, 64, 64, None) == 1
    # empty
    assert L.dequant_f16(1, None, None, 0, 256, 256, None) == 0
    assert L.dequant_f16(2, None, None, 4, 0, 0, None) == 0
    # prefill: K must be a multiple of the block width; unknown format
    assert L.prefill_f16(1, 4, 4, 32, 8, 32, 4096, 1 << 24, 1 << 26, 4, 1, 0, None, None, 0,
                         None) == 1
    assert L.prefill_f16(7, 4, 4, 256, 8, 256, 4096, 1 << 24, 1 << 26, 4, 1, 0, None, None, 0,
                         None) == 1
    assert L.prefill_f16(2, 0, 4, 256, 8, 256, 4096, 1 << 24, 1 << 26, 4, 1, 0, None, None, 0,
                         None) == 0


def test_workspace_sizes():
    assert dge.gemm_workspace_size_splits(100, 50, 1) == 0
    assert dge.gemm_workspace_size_splits(100, 50, 3) == 3 * 100 * 50 * 4
    assert dge.gemm_workspace_size(0, 5, 5) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="pins the 256-CU choices")
def test_fp32_schedule_choices():
    # the fp32 model (FLOPs of the busiest CU at each tile's rate): 1024^3
    # splits K in two (128 x 64 tiles fill only half the CUs), 2048^3 and
    # 4096^3 fill the CUs without a split
    f32 = torch.float32
    assert dge.gemm_workspace_size(1024, 1024, 1024, f32) == 2 * 1024 * 1024 * 4
    assert dge.gemm_workspace_size(2048, 2048, 2048, f32) == 0
    assert dge.gemm_workspace_size(4096, 4096, 4096, f32) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_no_device_reports_device_error():
    assert dge.lib().gemm_init() == 5
    assert _call(dge.lib()) == 5


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_forced_failure_hook(monkeypatch):
    monkeypatch.setenv("GEMM_TEST_FAIL", "launch")
    assert _call(dge.lib()) == 4
    monkeypatch.setenv("GEMM_TEST_FAIL", "workspace")
    assert _call(dge.lib()) == 3
    monkeypatch.setenv("GEMM_TEST_FAIL", "launch")
    assert _call(dge.lib(), M=-1) == 1  # validation first
