"""fp8_quantize_tensor_current_noalloc (the library's static scratch, no
workspace, nothing allocated) against fp8_quantize_tensor_current with a
caller-owned workspace, through the C ABI: FP8 bytes, transposed bytes,
amax and the scale pair bit for bit, on two calls in a row on one stream,
the second with a smaller input (the scratch keeps the first call's
contents).  The cases cover the one-launch path, the two-launch path with
a transposed copy, and a tensor too large for one launch; the first pair is
also checked against the oracle."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import DEV, bytes8, dev_bf16, f32
from tests.test_gpu_quant import rand_bits

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


def _outs(shape, transposed):
    R, C = shape
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((C, R), dtype=torch.uint8, device=DEV) if transposed else None
    return [q, qT] + [torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
                      for _ in range(3)]


def _snap(o):
    return [None if t is None else (bytes8(t) if t.dtype == torch.uint8 else
                                    f32(t).view(np.uint32)) for t in o]


@pytest.mark.parametrize("first,second,transposed,fmt", [
    ((4096, 8192), (1000, 1008), False, E4M3),     # one launch, then a smaller one
    ((4112, 8208), (272, 384), True, E5M2),        # amax pass + cast with qT, twice
    ((6400, 8192), (64, 64), False, E4M3),         # too large for one launch, then tiny
])
def test_noalloc_matches_workspace_call(F, orc, first, second, transposed, fmt):
    ws = F.workspace()
    for call, shape in enumerate((first, second)):
        x = rand_bits(shape, 40 + call + shape[1], 2.0, specials=True)
        xd = dev_bf16(x)
        got, want = _outs(shape, transposed), _outs(shape, transposed)
        print(f"noalloc call {call}: {shape} qT={transposed} fmt={fmt}", flush=True)
        F.fp8_quantize_tensor_current_noalloc(xd, fmt, *got)
        F.fp8_quantize_tensor_current(xd, fmt, *want, workspace=ws)
        torch.cuda.synchronize()
        g, w = _snap(got), _snap(want)
        for name, a, b in zip(("q", "qT", "amax", "scale", "scale_inv"), g, w):
            if a is None:
                continue
            assert np.array_equal(a, b), f"call {call} {shape}: {name} differs"
        if call == 0 and first == (4096, 8192):
            wa = orc.amax(x)
            s, si = orc.scale_from_amax(wa, fmt)
            assert g[2][0] == np.float32(wa).view(np.uint32)
            assert g[4][0] == np.float32(si).view(np.uint32)
            wq, _, _ = orc.quantize_tensor(x, fmt, s)
            assert np.array_equal(g[0], wq)


def test_noalloc_rejects_bad_arguments_before_touching_the_scratch(F):
    L = F.lib()
    P = 0x10000
    assert L.fp8_quantize_tensor_current_noalloc(P, 4, 16, 0, P, None, None, None, P, None) == 1
    assert L.fp8_quantize_tensor_current_noalloc(P, 4, 24, 0, P, None, P, None, P, None) == 3
    assert L.fp8_quantize_tensor_current_noalloc(P, 4, 16, 9, P, None, P, None, P, None) == 4
    assert L.fp8_quantize_tensor_current_noalloc(P, -4, 16, 0, P, None, P, None, P, None) == 2
