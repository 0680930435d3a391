"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/fp8sg.h declares, and rejects bad arguments with the
documented status before anything is launched (the pointers below are never
dereferenced: every call fails validation on the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8sg.h")

OK, NULL, SHAPE, ALIGN, UNSUP, HIP = 0, 1, 2, 3, 4, 5
P = 0x10000          # a 16-byte-aligned fake device address
PU = 0x10001         # a misaligned one


@pytest.fixture(scope="module")
def L():
    from scaled_fp8_gemm_amd import fp8sg
    return fp8sg.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:fp8_status_t|const char\*)\s+(fp8_\w+)\(", text, re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    from scaled_fp8_gemm_amd import fp8sg
    for code, name in fp8sg.STATUS.items():
        assert fp8sg.fp8_status_string(code).startswith(name)


def test_amax_errors(L):
    assert L.fp8_amax(None, 4, 16, 0, P, None, None, P, None) == NULL
    assert L.fp8_amax(P, 4, 16, 0, None, None, None, P, None) == NULL
    assert L.fp8_amax(P, 4, 16, 0, P, None, None, None, None) == NULL     # workspace
    assert L.fp8_amax(P, 4, 16, 7, P, None, None, P, None) == UNSUP
    assert L.fp8_amax(P, -1, 16, 0, P, None, None, P, None) == SHAPE
    assert L.fp8_amax(PU, 4, 16, 0, P, None, None, P, None) == ALIGN
    assert L.fp8_amax(P, 4, 16, 0, P + 2, None, None, P, None) == ALIGN
    assert L.fp8_amax(P, 4, 16, 0, P, None, None, P + 128, None) == ALIGN  # workspace % 256


def test_workspace_init_errors(L):
    from scaled_fp8_gemm_amd import fp8sg
    assert fp8sg.WORKSPACE_BYTES == int(re.search(r"#define FP8_WORKSPACE_BYTES (\d+)",
                                                  open(HEADER).read()).group(1))
    w = L.fp8_workspace_init
    assert w(None, 0, None) == NULL
    assert w(P, -1, None) == SHAPE
    assert w(P + 16, 0, None) == ALIGN


def test_quantize_tensor_errors(L):
    q = L.fp8_quantize_tensor
    assert q(None, 4, 16, 0, P, P, None, None, None, None) == NULL
    assert q(P, 4, 16, 0, None, P, None, None, None, None) == NULL
    assert q(P, 4, 16, 0, P, None, None, None, None, None) == NULL
    assert q(P, 4, 16, 2, P, P, None, None, None, None) == UNSUP
    assert q(P, 4, -16, 0, P, P, None, None, None, None) == SHAPE
    assert q(P, 4, 24, 0, P, P, None, None, None, None) == ALIGN          # cols % 16
    assert q(P, 8, 16, 0, P, P, P, None, None, None) == ALIGN             # qT needs rows % 16
    assert q(PU, 16, 16, 0, P, P, None, None, None, None) == ALIGN
    assert q(P, 16, 16, 0, P, P, None, P, None, None) == NULL       # amax_out needs a workspace
    assert q(P, 16, 16, 0, P, P, None, P, P + 64, None) == ALIGN


def test_history_errors(L):
    h = L.fp8_amax_history_update
    assert h(None, 16, 0, P, 0, P, P, None) == NULL
    assert h(P, 16, 0, P, 0, None, P, None) == NULL
    assert h(P, 0, 0, P, 0, P, P, None) == SHAPE
    assert h(P, 1025, 0, P, 0, P, P, None) == SHAPE
    assert h(P, 16, -1, P, 0, P, P, None) == SHAPE
    assert h(P, 16, 0, P, 5, P, P, None) == UNSUP


def test_block_and_mx_errors(L):
    b = L.fp8_quantize_block
    assert b(P, 128, 256, 0, 2, 128, P, P, None) == UNSUP            # block_rows
    assert b(P, 128, 256, 0, 1, 64, P, P, None) == UNSUP             # block_cols
    assert b(P, 128, 200, 0, 1, 128, P, P, None) == SHAPE            # cols % 128
    assert b(P, 100, 256, 0, 128, 128, P, P, None) == SHAPE          # rows % 128
    assert b(None, 128, 256, 0, 1, 128, P, P, None) == NULL
    m = L.fp8_quantize_mx
    assert m(P, 4, 48, 0, P, P, None) == SHAPE                        # cols % 32
    assert m(P, 4, 64, 0, None, P, None) == NULL
    assert m(PU, 4, 64, 0, P, P, None) == ALIGN


def test_quantize_current_errors(L):
    c = L.fp8_quantize_tensor_current
    assert c(P, 4, 16, 0, P, None, None, None, P, P, None) == NULL     # amax
    assert c(P, 4, 16, 0, P, None, P, None, None, P, None) == NULL     # scale_inv
    assert c(P, 4, 16, 0, P, None, P, None, P, None, None) == NULL     # workspace
    assert c(P, 4, 24, 0, P, None, P, None, P, P, None) == ALIGN       # cols % 16
    assert c(P, 8, 16, 0, P, P, P, None, P, P, None) == ALIGN          # qT rows % 16
    assert c(P, 4, 16, 0, P, None, P, None, P, P + 16, None) == ALIGN  # workspace % 256
    assert c(P, 4, 16, 2, P, None, P, None, P, P, None) == UNSUP


def test_quantize_pair_current_errors(L):
    c = L.fp8_quantize_pair_current
    good = (P, 4, 16, 0, P, P, None, P)
    assert c(P, 4, 16, 0, P, None, None, P, *good, P, None) == NULL        # a's amax
    assert c(*good, P, 4, 16, 0, P, P, None, None, P, None) == NULL        # b's scale_inv
    assert c(None, 4, 16, 0, P, P, None, P, *good, P, None) == NULL        # a's input
    assert c(*good, P, 4, 16, 0, None, P, None, P, P, None) == NULL        # b's output
    assert c(P, -1, 16, 0, P, P, None, P, *good, P, None) == SHAPE
    assert c(*good, P, 4, 24, 0, P, P, None, P, P, None) == ALIGN          # b's cols % 16
    assert c(PU, 4, 16, 0, P, P, None, P, *good, P, None) == ALIGN
    assert c(*good, P, 4, 16, 0, P, P, PU, P, P, None) == ALIGN            # b's scale
    assert c(P, 4, 16, 2, P, P, None, P, *good, P, None) == UNSUP
    assert c(*good, P, 4, 16, 5, P, P, None, P, P, None) == UNSUP
    assert c(P, 4, 16, 0, P, P, None, P, *good, None, None) == NULL     # workspace
    # a is checked before b
    assert c(P, 4, 16, 2, P, P, None, P, P, 4, 24, 0, P, P, None, P, P, None) == UNSUP


def test_f32_input_errors(L):
    a = L.fp8_amax_f32
    assert a(P, 4, 16, 0, None, None, None, P, None) == NULL
    assert a(P, 4, 16, 0, P, None, None, None, None) == NULL             # workspace
    assert a(P, -1, 16, 0, P, None, None, P, None) == SHAPE
    assert a(PU, 4, 16, 0, P, None, None, P, None) == ALIGN
    assert a(P, 4, 16, 3, P, None, None, P, None) == UNSUP
    q = L.fp8_quantize_tensor_f32
    assert q(P, 4, 24, 0, P, P, None, None, None, None) == ALIGN         # cols % 16
    assert q(P, 8, 16, 0, P, P, P, None, None, None) == ALIGN            # qT needs rows % 16
    assert q(None, 4, 16, 0, P, P, None, None, None, None) == NULL
    assert q(P, 16, 16, 0, P, P, None, P, None, None) == NULL            # amax_out, no workspace


def test_transposed_block_and_mx_errors(L):
    bt = L.fp8_quantize_block_t
    assert bt(P, 128, 256, 0, 2, P, P, P, P, None) == UNSUP           # block_rows
    assert bt(P, 100, 256, 0, 1, P, P, P, P, None) == SHAPE           # rows % 128
    assert bt(P, 128, 200, 0, 128, P, P, P, P, None) == SHAPE         # cols % 128
    assert bt(P, 128, 256, 0, 1, P, None, P, P, None) == NULL         # q without scale_inv
    assert bt(P, 128, 256, 0, 1, None, None, None, P, None) == NULL   # qT required
    assert bt(P, 128, 256, 0, 1, None, None, P, None, None) == NULL
    assert bt(P, 128, 256, 0, 1, None, None, PU, P, None) == ALIGN
    assert bt(P, 128, 256, 2, 1, None, None, P, P, None) == UNSUP     # fmt
    mt = L.fp8_quantize_mx_t
    assert mt(P, 48, 64, 0, P, P, P, P, None) == SHAPE                # rows % 32
    assert mt(P, 64, 48, 0, P, P, P, P, None) == SHAPE                # cols % 32
    assert mt(P, 64, 64, 0, None, P, P, P, None) == NULL
    assert mt(P, 64, 64, 0, None, None, None, P, None) == NULL
    assert mt(PU, 64, 64, 0, None, None, P, P, None) == ALIGN


def _op(fmt, scaling, data=P, s=P):
    from scaled_fp8_gemm_amd import fp8sg
    return fp8sg.Operand(data, fmt, scaling, s)


def test_gemm_errors(L):
    g = L.fp8_gemm_fprop
    r = ctypes.byref
    t = _op(0, 0)
    assert g(None, r(t), 16, 16, 16, P, None) == NULL
    assert g(r(t), r(t), 16, 16, 16, None, None) == NULL
    assert g(r(_op(0, 0, data=None)), r(t), 16, 16, 16, P, None) == NULL
    assert g(r(_op(0, 0, s=None)), r(t), 16, 16, 16, P, None) == NULL
    assert g(r(_op(3, 0)), r(t), 16, 16, 16, P, None) == UNSUP
    assert g(r(_op(0, 9)), r(t), 16, 16, 16, P, None) == UNSUP
    assert g(r(_op(0, 1)), r(t), 16, 16, 128, P, None) == UNSUP       # block x tensor
    assert g(r(_op(0, 3)), r(_op(0, 1)), 16, 16, 128, P, None) == UNSUP
    assert g(r(t), r(t), -1, 16, 16, P, None) == SHAPE
    assert g(r(t), r(t), 16, 16, 24, P, None) == ALIGN                # K % 16
    assert g(r(_op(0, 1)), r(_op(0, 2)), 16, 128, 64, P, None) == SHAPE   # K % 128
    assert g(r(_op(0, 1)), r(_op(0, 2)), 16, 100, 128, P, None) == SHAPE  # 128x128 rows
    assert g(r(_op(0, 3)), r(_op(0, 3)), 16, 16, 48, P, None) == SHAPE    # K % 32
    assert g(r(t), r(t), 16, 16, (1 << 23) + 16, P, None) == SHAPE        # K > 2^23
    assert g(r(t), r(t), 16, 16, 16, PU, None) == ALIGN
    assert g(r(_op(0, 0, data=PU)), r(t), 16, 16, 16, P, None) == ALIGN
    ff = L.fp8_gemm_fprop_fused
    assert ff(r(t), r(t), 16, 16, 16, P, 0, P, None, None, None, None) == NULL   # nothing fused
    assert ff(r(t), r(t), 16, 16, 16, P, 0, None, P, None, None, None) == NULL   # y_q, no scale
    assert ff(r(t), r(t), 16, 16, 16, P, 5, P, P, None, None, None) == UNSUP     # y_fmt
    assert ff(r(t), r(t), 16, 24, 16, P, 0, P, P, None, None, None) == ALIGN     # N % 16
    assert ff(r(t), r(t), 16, 16, 16, None, 0, P, None, P, P, None) == NULL      # amax only, no y
    assert ff(r(t), r(t), 16, 16, 16, P, 0, None, None, P, None, None) == NULL   # amax, no ws
    assert ff(r(t), r(t), 16, 16, 16, P, 0, None, None, P, P + 32, None) == ALIGN
    wf = L.fp8_gemm_wgrad_f32
    assert wf(r(t), r(t), 16, 16, 16, P, 2, None) == UNSUP             # accumulate flag
    assert wf(r(t), r(t), 24, 16, 16, P, 0, None) == ALIGN             # M % 16
    assert wf(r(t), r(t), 16, 16, 16, None, 1, None) == NULL
    # dgrad contracts over N, wgrad over M
    assert L.fp8_gemm_dgrad(r(t), r(t), 16, 24, 16, P, None) == ALIGN
    assert L.fp8_gemm_wgrad(r(t), r(t), 24, 16, 16, P, None) == ALIGN


def test_convert_errors(L):
    c = L.fp8_convert_f32
    assert c(None, 4, 0, P, None) == NULL
    assert c(P, -1, 0, P, None) == SHAPE
    assert c(P, 4, 3, P, None) == UNSUP
    assert c(PU, 4, 0, P, None) == ALIGN


def test_plain_c_caller(tmp_path):
    """A C99 program (tests/c_abi_check.c) includes the header with no HIP or
    torch headers, links the library and gets the documented statuses from
    its validation, before anything reaches a device."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    lib_dir = os.path.join(ROOT, "scaled_fp8_gemm_amd")
    exe = str(tmp_path / "c_abi_check")
    subprocess.check_call([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c_abi_check.c"),
                           "-L", lib_dir, "-lfp8sg", f"-Wl,-rpath,{lib_dir}", "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout


def test_operand_keeps_its_tensors():
    """fp8sg.operand holds the tensors it points at, so temporaries passed to
    it (say operand(torch.from_numpy(a).to(dev), ...)) are not freed, and
    their memory reused, before the GEMM call is enqueued."""
    import gc
    import weakref

    import torch
    from scaled_fp8_gemm_amd import fp8sg
    data, scale = torch.zeros(64, dtype=torch.uint8), torch.ones(1)
    refs = (weakref.ref(data), weakref.ref(scale))
    o = fp8sg.operand(data, fp8sg.E4M3, fp8sg.SCALE_TENSOR, scale)
    del data, scale
    gc.collect()
    assert all(r() is not None for r in refs)
    assert o.data == refs[0]().data_ptr() and o.scale_inv == refs[1]().data_ptr()
    del o
    gc.collect()
    assert all(r() is None for r in refs)
