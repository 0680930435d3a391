"""GPU parity of the quantise path: amax, scale pair, per-tensor cast (with
transposed copy and fused amax), delayed-scaling history, blockwise and MX
casts.  Every byte, scale and amax must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import DEV, bits16, bytes8, dev_bf16, dev_f32, f32

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


def rand_bits(shape, seed, scale=1.0, specials=False):
    """BF16 bit patterns: scaled normals, optionally sprinkled with specials."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    b = ((f.view(np.uint32) + 0x7FFF + ((f.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    if specials and b.size >= 16:
        flat = b.reshape(-1)
        idx = rng.choice(flat.size, size=min(64, flat.size // 4), replace=False)
        pool = np.array([0x0000, 0x8000, 0x0001, 0x8003, 0x007F, 0x7F7F, 0xFF7F, 0x3F80],
                        np.uint16)
        flat[idx] = pool[rng.integers(0, pool.size, size=idx.size)]
    return b


def empty_dev(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


# (2056, 8208) spans more 16 KB chunks than the launch has workgroups, with a
# ragged last chunk.
@pytest.mark.parametrize("shape", [(0, 0), (1, 1), (3, 5), (37, 41), (1000, 1000), (4096, 513),
                                   (2056, 8208)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_amax_and_scale(F, orc, shape, fmt):
    x = rand_bits(shape, 1 + shape[0], 3.0, specials=True)
    xd = dev_bf16(x) if x.size else torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
    F.fp8_amax(xd, fmt, am, s, si)
    want = orc.amax(x) if x.size else 0.0
    ws, wsi = orc.scale_from_amax(want, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(want).view(np.uint32)
    assert f32(s)[0] == ws and f32(si)[0] == wsi


def test_amax_special_values(F, orc):
    for special, expect_nan in ((0x7FC0, True), (0xFF80, False), (0x7F80, False)):
        x = rand_bits((64, 64), 5)
        x[10, 20] = special
        am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
        F.fp8_amax(dev_bf16(x), E4M3, am, s, si)
        a = f32(am)[0]
        assert np.isnan(a) == expect_nan and (expect_nan or np.isinf(a))
        assert f32(s)[0] == 1.0 and f32(si)[0] == 1.0
    # a BF16-subnormal amax: the quotient overflows and the scale clamps
    x = np.zeros((8, 16), np.uint16)
    x[3, 3] = 0x0001
    am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
    F.fp8_amax(dev_bf16(x), E4M3, am, s, si)
    ws, wsi = orc.scale_from_amax(orc.amax(x), E4M3)
    assert f32(s)[0] == ws == np.finfo(np.float32).max and f32(si)[0] == wsi


@pytest.mark.parametrize("shape,transposed", [((0, 16), False), ((1, 16), False),
                                              ((37, 48), False), ((48, 400), True),
                                              ((256, 256), True), ((272, 384), True),
                                              ((2000, 1040), True), ((3, 4096), False),
                                              # more chunks / tiles than workgroups, ragged
                                              ((4112, 8208), False), ((4112, 8208), True)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("fused_amax", [False, True])
def test_quantize_tensor(F, orc, shape, transposed, fmt, fused_amax):
    x = rand_bits(shape, 7 + shape[1], 2.0, specials=True)
    xd = dev_bf16(x) if x.size else torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    # a scale that saturates the largest values (as delayed scaling can)
    scale = np.float32({E4M3: 448.0, E5M2: 57344.0}[fmt] / 3.0)
    R, C = shape
    q = empty_dev(shape, torch.uint8)
    qT = empty_dev((C, R), torch.uint8) if transposed else None
    am = empty_dev(1, torch.float32) if fused_amax else None
    F.fp8_quantize_tensor(xd, fmt, dev_f32([scale]), q, qT, am)
    wq, wqT, wam = orc.quantize_tensor(x, fmt, scale, transposed=transposed, want_amax=fused_amax)
    assert np.array_equal(bytes8(q), wq)
    if transposed:
        assert np.array_equal(bytes8(qT), wqT)
    if fused_amax:
        assert f32(am)[0].view(np.uint32) == np.float32(wam).view(np.uint32)


def test_history_sequence(F, orc):
    H = 16
    hist_d = torch.zeros(H, dtype=torch.float32, device=DEV)
    hist = np.zeros(H, np.float32)
    s, si = empty_dev(1, torch.float32), empty_dev(1, torch.float32)
    rng = np.random.Generator(np.random.PCG64(3))
    for t in range(45):
        a = np.float32(rng.uniform(0.5, 100.0) if t != 7 else 5000.0)
        if t == 30:
            a = np.float32(np.nan)
        F.fp8_amax_history_update(hist_d, t, dev_f32([a]), E5M2 if t % 2 else E4M3, s, si)
        ws, wsi = orc.amax_history_update(hist, t, a, E5M2 if t % 2 else E4M3)
        got = f32(hist_d)
        assert np.array_equal(got.view(np.uint32), hist.view(np.uint32)), t
        assert f32(s)[0] == ws and f32(si)[0] == wsi, t


@pytest.mark.parametrize("shape,br", [((256, 384), 1), ((256, 384), 128), ((1, 128), 1),
                                      ((384, 1024), 128), ((0, 256), 1), ((999, 640), 1),
                                      ((2056, 8192), 1)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_block(F, orc, shape, br, fmt):
    x = rand_bits(shape, 11 + shape[0], 1.0, specials=True)
    if x.size:
        x[0, :128] = 0                                 # an all-zero tile
    xd = dev_bf16(x) if x.size else torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    R, C = shape
    q = empty_dev(shape, torch.uint8)
    si = empty_dev((R // br, C // 128), torch.float32)
    F.fp8_quantize_block(xd, fmt, br, 128, q, si)
    if x.size == 0:
        return
    wq, wsi = orc.quantize_block(x, fmt, br, 128)
    assert np.array_equal(bytes8(q), wq)
    assert np.array_equal(f32(si).view(np.uint32), wsi.view(np.uint32))


@pytest.mark.parametrize("shape", [(1, 32), (33, 96), (128, 4096), (257, 1024), (2056, 8192)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_mx(F, orc, shape, fmt):
    x = rand_bits(shape, 13 + shape[0], 4.0, specials=True)
    R, C = shape
    if R > 4:
        x[1, 0:32] = 0                                 # zero block -> 127
        x[2, 32] = 0x7FC0                              # NaN block -> 0xFF
        x[3, 0:32] = 0x0001                            # BF16-subnormal block -> clamp -127
        x[4, 0:32] = 0x7F7F                            # largest BF16 -> e = 120
        x[4, 40] = 0xFF80                              # -inf block
    q = empty_dev(shape, torch.uint8)
    e = empty_dev((R, C // 32), torch.uint8)
    F.fp8_quantize_mx(dev_bf16(x), fmt, q, e)
    wq, we = orc.quantize_mx(x, fmt)
    assert np.array_equal(bytes8(e), we)
    assert np.array_equal(bytes8(q), wq)


@pytest.mark.parametrize("shape,transposed", [((0, 16), False), ((1, 16), False),
                                              ((37, 48), False), ((272, 384), True),
                                              ((3072, 8192), False), ((4112, 8208), False),
                                              ((4112, 8208), True), ((6400, 8192), False)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_tensor_current(F, orc, shape, transposed, fmt):
    """One-call current scaling = fp8_amax + fp8_quantize_tensor, bit for bit,
    and the oracle's amax / scale rule / cast.  The shapes cover the one-launch
    path at both register budgets (256 bytes per thread: 1x16, 37x48,
    3072x8192 and 4112x8208; 384 bytes: the 11008x4096 weight in the workload
    tests) and the two-launch fallbacks (transposed copy; 6400x8192, more than
    the registers of a co-resident grid hold)."""
    x = rand_bits(shape, 101 + shape[1], 2.0, specials=True)
    xd = dev_bf16(x) if x.size else torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    R, C = shape
    q = empty_dev(shape, torch.uint8)
    qT = empty_dev((C, R), torch.uint8) if transposed else None
    am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
    F.fp8_quantize_tensor_current(xd, fmt, q, qT, am, s, si)
    wa = orc.amax(x) if x.size else 0.0
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32)
    assert f32(s)[0] == ws and f32(si)[0] == wsi
    if x.size == 0:
        return
    wq, wqT, _ = orc.quantize_tensor(x, fmt, ws, transposed=transposed)
    assert np.array_equal(bytes8(q), wq)
    if transposed:
        assert np.array_equal(bytes8(qT), wqT)


def test_quantize_tensor_current_concurrent_streams(F, orc):
    """Two one-launch current-scaling calls running at once on different
    streams, each grid as large as the device holds.  However the two grids'
    workgroups interleave (one grid can keep the other from being resident),
    both results are the oracle's, bit for bit: when a grid-wide wait runs
    out, one workgroup completes the amax from the maxima already in and the
    inputs of the workgroups that have not arrived."""
    shape = (4096, 8192)
    xs = [rand_bits(shape, 700 + i, 3.0) for i in range(2)]
    dx = [dev_bf16(x) for x in xs]
    streams = [torch.cuda.Stream() for _ in xs]
    outs = [(empty_dev(shape, torch.uint8),) + tuple(empty_dev(1, torch.float32) for _ in range(3))
            for _ in xs]
    wss = [F.workspace() for _ in xs]            # one workspace per stream
    torch.cuda.synchronize()
    for _ in range(3):
        for x, st, (q, am, s, si), ws in zip(dx, streams, outs, wss):
            F.fp8_quantize_tensor_current(x, E4M3, q, None, am, s, si, stream=st, workspace=ws)
    torch.cuda.synchronize()
    for x, (q, am, s, si) in zip(xs, outs):
        wa = orc.amax(x)
        ws, wsi = orc.scale_from_amax(wa, E4M3)
        assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32)
        assert f32(s)[0] == ws and f32(si)[0] == wsi
        wq, _, _ = orc.quantize_tensor(x, E4M3, ws)
        assert np.array_equal(bytes8(q), wq)


def _current_outputs(shape):
    return (empty_dev(shape, torch.uint8),) + tuple(empty_dev(1, torch.float32) for _ in range(3))


def _check_current(orc, x, fmt, q, am, s, si, label):
    wa = orc.amax(x) if x.size else 0.0
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32), label
    assert f32(s)[0] == ws and f32(si)[0] == wsi, label
    if x.size:
        wq, _, _ = orc.quantize_tensor(x, fmt, ws)
        assert np.array_equal(bytes8(q), wq), label


# (4096, 4096) + (11008, 4096): the LLaMA2-7B up-projection's X and W, one
# launch; (8192, 8192) + (256, 256): more than the device holds at once, one
# call per tensor; (0, 16): an empty tensor.
@pytest.mark.parametrize("sa,sb,fa,fb", [
    ((1, 16), (37, 48), E4M3, E5M2),
    ((256, 256), (256, 256), E4M3, E4M3),
    ((4112, 8208), (272, 384), E5M2, E4M3),
    ((1000, 1008), (3000, 2064), E5M2, E5M2),
    ((4096, 4096), (11008, 4096), E4M3, E4M3),
    ((8192, 8192), (256, 256), E4M3, E4M3),
    ((0, 16), (37, 48), E4M3, E4M3),
])
def test_quantize_pair_current(F, orc, sa, sb, fa, fb):
    """Current scaling of two tensors in one call: each tensor's amax, scale
    pair and FP8 bytes are the oracle's, bit for bit.  Three calls in a row on
    one stream, the second with the tensors' data exchanged for fresh draws
    (one with a NaN) and a single-tensor call in between, so each call starts
    from the words the previous one left."""
    outs = (_current_outputs(sa), _current_outputs(sb))
    ws = F.workspace()
    for rep in range(3):
        xa = rand_bits(sa, 900 + 10 * rep + sa[1], 2.0, specials=True)
        xb = rand_bits(sb, 901 + 10 * rep + sb[1], 0.02, specials=True)
        if rep == 1 and xb.size:
            xb.reshape(-1)[xb.size // 2] = 0x7FC0                      # NaN: amax NaN, scale 1
        da = dev_bf16(xa) if xa.size else torch.empty(sa, dtype=torch.bfloat16, device=DEV)
        db = dev_bf16(xb) if xb.size else torch.empty(sb, dtype=torch.bfloat16, device=DEV)
        F.fp8_quantize_pair_current(da, fa, *outs[0], db, fb, *outs[1], workspace=ws)
        if rep == 1:
            one = _current_outputs((64, 64))
            x1 = rand_bits((64, 64), 77, 1.0)
            F.fp8_quantize_tensor_current(dev_bf16(x1), E4M3, one[0], None, *one[1:],
                                          workspace=ws)
        torch.cuda.synchronize()
        _check_current(orc, xa, fa, *outs[0], label=f"a rep {rep}")
        _check_current(orc, xb, fb, *outs[1], label=f"b rep {rep}")
        if rep == 1:
            _check_current(orc, x1, E4M3, *one, label="single")


def rand_f32(shape, seed, scale=1.0):
    """FP32 values with a wide magnitude range and a few specials."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = (rng.standard_normal(shape) * np.exp(rng.standard_normal(shape) * 2) * scale)
    f = f.astype(np.float32)
    if f.size >= 16:
        flat = f.reshape(-1)
        flat[1] = -0.0
        flat[2] = np.float32(1e-45)                           # FP32 subnormal
        flat[3] = np.float32(3.4e38)
    return f


# FP32 master weights: 4 elements per 16-byte vector, so the tails differ from BF16
@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (37, 41), (1000, 1003), (2056, 8208)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_amax_f32(F, orc, shape, fmt):
    x = rand_f32(shape, 81 + shape[0])
    am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
    F.fp8_amax_f32(torch.from_numpy(x).to(DEV), fmt, am, s, si)
    wa = orc.amax_f32(x)
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32)
    assert f32(s)[0] == ws and f32(si)[0] == wsi
    x[0, 0] = np.float32(np.nan)
    F.fp8_amax_f32(torch.from_numpy(x).to(DEV), fmt, am, s, si)
    assert np.isnan(f32(am)[0]) and f32(s)[0] == 1.0


@pytest.mark.parametrize("shape,transposed", [((1, 16), False), ((37, 48), False),
                                              ((48, 400), True), ((272, 384), True),
                                              ((4112, 8208), False), ((4112, 8208), True)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_tensor_f32(F, orc, shape, transposed, fmt):
    x = rand_f32(shape, 91 + shape[1], 10.0)
    R, C = shape
    xd = torch.from_numpy(x).to(DEV)
    s = torch.tensor([0.7310586], dtype=torch.float32, device=DEV)
    q = empty_dev(shape, torch.uint8)
    qT = empty_dev((C, R), torch.uint8) if transposed else None
    am = empty_dev(1, torch.float32)
    F.fp8_quantize_tensor_f32(xd, fmt, s, q, qT, am)
    wq, wqT, wam = orc.quantize_tensor_f32(x, fmt, f32(s)[0], transposed=transposed,
                                           want_amax=True)
    assert np.array_equal(bytes8(q), wq)
    if transposed:
        assert np.array_equal(bytes8(qT), wqT)
    assert f32(am)[0].view(np.uint32) == np.float32(wam).view(np.uint32)


def _specials_in_columns(x):
    """An all-zero column tile, a NaN, a -inf and a largest-BF16 entry in the
    first column tile, so column scales meet every special case."""
    R, C = x.shape
    x[:, 5] = 0
    x[7, 9] = 0x7FC0
    x[min(130, R - 1), 11 % C] = 0xFF80
    x[3, 13 % C] = 0x7F7F


# (4224, 8192): 2112 tiles of 128 x 128, more than the launch's workgroups
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 1024), (4224, 8192)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rowwise", [True, False])
def test_quantize_block_t_1x128(F, orc, shape, fmt, rowwise):
    """Row-wise 1x128 copy and the column-wise copy of x^T (128-row tiles)."""
    R, C = shape
    x = rand_bits(shape, 17 + R, 1.0, specials=True)
    _specials_in_columns(x)
    xd = dev_bf16(x)
    q = empty_dev(shape, torch.uint8) if rowwise else None
    si = empty_dev((R, C // 128), torch.float32) if rowwise else None
    qT = empty_dev((C, R), torch.uint8)
    siT = empty_dev((C, R // 128), torch.float32)
    F.fp8_quantize_block_t(xd, fmt, 1, q, si, qT, siT)
    wqT, wsiT = orc.quantize_block(np.ascontiguousarray(x.T), fmt, 1, 128)
    assert np.array_equal(f32(siT).view(np.uint32), wsiT.view(np.uint32))
    assert np.array_equal(bytes8(qT), wqT)
    if rowwise:
        wq, wsi = orc.quantize_block(x, fmt, 1, 128)
        assert np.array_equal(f32(si).view(np.uint32), wsi.view(np.uint32))
        assert np.array_equal(bytes8(q), wq)


@pytest.mark.parametrize("shape", [(128, 128), (384, 256), (1280, 2304)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_block_t_128(F, orc, shape, fmt):
    """128x128 blocks: the transposed copy is q^T with the transposed grid."""
    R, C = shape
    x = rand_bits(shape, 19 + R, 0.02, specials=True)
    _specials_in_columns(x)
    q = empty_dev(shape, torch.uint8)
    si = empty_dev((R // 128, C // 128), torch.float32)
    qT = empty_dev((C, R), torch.uint8)
    siT = empty_dev((C // 128, R // 128), torch.float32)
    F.fp8_quantize_block_t(dev_bf16(x), fmt, 128, q, si, qT, siT)
    wq, wsi = orc.quantize_block(x, fmt, 128, 128)
    assert np.array_equal(bytes8(q), wq)
    assert np.array_equal(f32(si).view(np.uint32), wsi.view(np.uint32))
    assert np.array_equal(bytes8(qT), np.ascontiguousarray(wq.T))
    assert np.array_equal(f32(siT).view(np.uint32), np.ascontiguousarray(wsi.T).view(np.uint32))


# ragged edge tiles (96 x 160, 160 x 96) and more tiles than workgroups
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (160, 96), (4224, 8224)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rowwise", [True, False])
def test_quantize_mx_t(F, orc, shape, fmt, rowwise):
    """Row-wise 1x32 MX copy and the column-wise copy of x^T (32-row blocks)."""
    R, C = shape
    x = rand_bits(shape, 23 + R, 4.0, specials=True)
    x[0:32, 1] = 0                                     # zero column block -> 127
    x[2, 3] = 0x7FC0                                   # NaN -> 0xFF
    x[0:32, 4] = 0x0001                                # subnormal block -> clamp -127
    x[0:32, 6] = 0x7F7F                                # largest BF16 -> e = 120
    x[5, 7] = 0xFF80                                   # -inf -> 0xFF
    q = empty_dev(shape, torch.uint8) if rowwise else None
    e = empty_dev((R, C // 32), torch.uint8) if rowwise else None
    qT = empty_dev((C, R), torch.uint8)
    eT = empty_dev((C, R // 32), torch.uint8)
    F.fp8_quantize_mx_t(dev_bf16(x), fmt, q, e, qT, eT)
    wqT, weT = orc.quantize_mx(np.ascontiguousarray(x.T), fmt)
    assert np.array_equal(bytes8(eT), weT)
    assert np.array_equal(bytes8(qT), wqT)
    if rowwise:
        wq, we = orc.quantize_mx(x, fmt)
        assert np.array_equal(bytes8(e), we)
        assert np.array_equal(bytes8(q), wq)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_convert_every_fp32_pattern(F, orc, fmt):
    """The cast's rounding routine on all 2^32 FP32 inputs, in 2^28 chunks."""
    chunk = 1 << 28
    base = torch.arange(chunk, dtype=torch.int64, device=DEV)
    q = empty_dev(chunk, torch.uint8)
    for lo in range(0, 1 << 32, chunk):
        x = (base + lo).to(torch.int32) if lo + chunk <= (1 << 31) else \
            (base + lo - (1 << 32)).to(torch.int32)
        F.fp8_convert_f32(x.view(torch.float32), fmt, q)
        got = bytes8(q)
        want = orc.encode_bits_range(lo, lo + chunk, fmt)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"fmt {fmt}: {bad.size} mismatches in chunk {lo:#x}, first input "
                               f"{lo + int(bad[0]):#010x}: gpu {got[bad[0]]:#04x} "
                               f"oracle {want[bad[0]]:#04x}")
    # ragged tail path (n % 4 != 0)
    x = torch.tensor([1.0, -2.5, 1e9, float("nan"), 3e-3, -0.0, 7.0], device=DEV)
    q = empty_dev(7, torch.uint8)
    F.fp8_convert_f32(x, fmt, q)
    assert np.array_equal(bytes8(q), orc.encode(x.cpu().numpy(), fmt))


def test_quantise_beyond_2_31_elements(F, orc):
    """Maximum sizes: a BF16 tensor of 65552 x 32768 = 2^31 + 2^19 elements
    (4.3 GB), so element indices and byte offsets pass 2^31.  Current scaling
    (two launches at this size), the transposed copy, 1x128 blocks and MX
    blocks are each the oracle's, bit for bit; the largest magnitude sits
    beyond element 2^31."""
    R, C = 65552, 32768
    n = R * C
    rng = np.random.Generator(np.random.PCG64(31))
    x = rng.integers(0, 2 ** 32, size=n // 2, dtype=np.uint32).view(np.uint16)
    x &= 0xBFFF                                  # |x| < 2: finite, with subnormals
    x[(1 << 31) + 12345] = 0x4120                # 10.0, the amax, past 2^31
    x = x.reshape(R, C)
    xd = dev_bf16(x)
    fmt = E4M3

    am, s, si = (empty_dev(1, torch.float32) for _ in range(3))
    q = empty_dev((R, C), torch.uint8)
    F.fp8_quantize_tensor_current(xd, fmt, q, None, am, s, si)
    torch.cuda.synchronize()
    wa = orc.amax(x)
    assert wa == 10.0
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0] == wa and f32(s)[0] == ws and f32(si)[0] == wsi
    wq, wqT, _ = orc.quantize_tensor(x, fmt, ws, transposed=True)
    assert np.array_equal(bytes8(q), wq)

    qT = empty_dev((C, R), torch.uint8)
    q.zero_()
    F.fp8_quantize_tensor(xd, fmt, s, q, qT)
    torch.cuda.synchronize()
    assert np.array_equal(bytes8(q), wq)
    del wq
    assert np.array_equal(bytes8(qT), wqT)
    del wqT, qT

    sb = empty_dev((R, C // 128), torch.float32)
    F.fp8_quantize_block(xd, fmt, 1, 128, q, sb)
    torch.cuda.synchronize()
    bq, bs = orc.quantize_block(x, fmt, 1, 128)
    assert np.array_equal(f32(sb).view(np.uint32), bs.view(np.uint32))
    assert np.array_equal(bytes8(q), bq)
    del bq, bs, sb

    e = empty_dev((R, C // 32), torch.uint8)
    F.fp8_quantize_mx(xd, fmt, q, e)
    torch.cuda.synchronize()
    mq, me = orc.quantize_mx(x, fmt)
    assert np.array_equal(bytes8(e), me)
    assert np.array_equal(bytes8(q), mq)


def test_quantize_pair_current_concurrent_streams(F, orc):
    """Two paired one-launch calls running at once on different streams, each
    grid as large as the device holds (the LLaMA2-7B up-projection's X and W):
    however the grids interleave, every tensor's amax, scale pair and bytes
    are the oracle's (when a grid-wide wait runs out, one workgroup completes
    the amax from the maxima already in and the inputs of the workgroups that
    have not arrived, and publishes it)."""
    shapes = ((4096, 4096), (11008, 4096))
    xs = [[rand_bits(sh, 800 + 10 * i + j, 2.0 if j == 0 else 0.02) for j, sh in enumerate(shapes)]
          for i in range(2)]
    dx = [[dev_bf16(x) for x in pair] for pair in xs]
    outs = [[_current_outputs(sh) for sh in shapes] for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    wss = [F.workspace() for _ in range(2)]      # one workspace per stream
    torch.cuda.synchronize()
    for _ in range(3):
        for d, o, st, ws in zip(dx, outs, streams, wss):
            F.fp8_quantize_pair_current(d[0], E4M3, *o[0], d[1], E4M3, *o[1], stream=st,
                                        workspace=ws)
    torch.cuda.synchronize()
    for i in range(2):
        for j in range(2):
            _check_current(orc, xs[i][j], E4M3, *outs[i][j], label=f"stream {i} tensor {j}")


@pytest.mark.parametrize("spike", [None, "first", "middle", "last"])
@pytest.mark.parametrize("calls", ["one", "pair"])
def test_current_scaling_wait_bound_fallback(F, orc, calls, spike):
    """The one-launch current scaling with its grid-wide wait bounded to one
    poll (fp8_workspace_init's wait_polls = 1): workgroups give up waiting
    almost at once, and the first of them completes the amax itself from the
    maxima already in and the inputs of the workgroups that have not arrived
    (or takes the published amax if all arrive meanwhile).  The results are
    still the oracle's, bit for bit, over three calls in a row on one
    workspace (the words each call leaves are consistent), also when one
    element far above the rest sits in the first, a middle or the last
    workgroup's share; a workspace with the default bound then gives the same
    bytes."""
    shapes = ((4096, 4096), (11008, 4096))
    xs = [rand_bits(sh, 950 + j, 2.0 if j == 0 else 0.02) for j, sh in enumerate(shapes)]
    if spike is not None:
        for j, x in enumerate(xs):
            flat = x.reshape(-1)
            at = {"first": 5, "middle": flat.size // 2 + 77, "last": flat.size - 3}[spike]
            # -300 and 3 are exact in BF16: the upper half of their FP32 bits
            flat[at] = np.array([-300.0 if j == 0 else 3.0], np.float32).view(np.uint32)[0] >> 16
    dx = [dev_bf16(x) for x in xs]
    ws1 = F.workspace(wait_polls=1)
    for rep in range(3):
        outs = [_current_outputs(sh) for sh in shapes]
        if calls == "pair":
            F.fp8_quantize_pair_current(dx[0], E4M3, *outs[0], dx[1], E4M3, *outs[1],
                                        workspace=ws1)
        else:
            for d, o in zip(dx, outs):
                F.fp8_quantize_tensor_current(d, E4M3, o[0], None, *o[1:], workspace=ws1)
        torch.cuda.synchronize()
        for j in range(2):
            _check_current(orc, xs[j], E4M3, *outs[j], label=f"{calls} rep {rep} tensor {j}")
            if spike is not None:
                assert f32(outs[j][1])[0] == (300.0 if j == 0 else 3.0), (spike, j)
    ref = [_current_outputs(sh) for sh in shapes]
    F.fp8_quantize_pair_current(dx[0], E4M3, *ref[0], dx[1], E4M3, *ref[1],
                                workspace=F.workspace())
    torch.cuda.synchronize()
    for j in range(2):
        assert np.array_equal(bytes8(ref[j][0]), bytes8(outs[j][0]))


# Workspace words of the one-launch grid-wide maximum (an internal layout,
# forged here to reach a state that 2^32 - 2 earlier calls would leave):
# set s starts at word 65536 + 4128 s; its top line at +4096 holds the
# publish claim [2], the rescue claim [3] and the generation [4]; group g's
# flag is the 64-bit word at +(64 + g) * 32 (low half amax, high half the
# generation that published it).
_GRID_AT, _SET_WORDS, _TOP_AT, _FLAG_AT = 65536, 4128, 4096, 64 * 32


def _forge_generation(ws, gen):
    words = ws.view(torch.int32)
    g = torch.tensor(np.array([gen], np.uint32).view(np.int32), device=DEV)
    for s in range(2):
        base = _GRID_AT + s * _SET_WORDS
        words[base + _TOP_AT + 2: base + _TOP_AT + 5] = g
        for grp in range(64):
            words[base + _FLAG_AT + grp * 32 + 1] = g    # published by generation G itself
    torch.cuda.synchronize()


@pytest.mark.parametrize("wait_polls", [0, 1])
@pytest.mark.parametrize("calls", ["one", "pair"])
def test_current_scaling_generation_wraps(F, orc, calls, wait_polls):
    """The grid-wide maximum tags flags and claims with a 32-bit generation
    that every call advances by one; calls across its wrap (0xFFFFFFFE ->
    0xFFFFFFFF -> 0 -> 1) give the oracle's bytes, with the default wait
    bound and with a one-poll bound (the rescue path), on one workspace."""
    shapes = ((4096, 4096), (11008, 4096))
    xs = [rand_bits(sh, 970 + j, 2.0 if j == 0 else 0.02) for j, sh in enumerate(shapes)]
    dx = [dev_bf16(x) for x in xs]
    ws = F.workspace(wait_polls=wait_polls)
    torch.cuda.synchronize()
    _forge_generation(ws, 0xFFFFFFFE)
    for rep in range(4):
        outs = [_current_outputs(sh) for sh in shapes]
        if calls == "pair":
            F.fp8_quantize_pair_current(dx[0], E4M3, *outs[0], dx[1], E4M3, *outs[1],
                                        workspace=ws)
        else:
            for d, o in zip(dx, outs):
                F.fp8_quantize_tensor_current(d, E4M3, o[0], None, *o[1:], workspace=ws)
        torch.cuda.synchronize()
        for j in range(2):
            _check_current(orc, xs[j], E4M3, *outs[j], label=f"{calls} wrap rep {rep} tensor {j}")
    # every call took the one-launch path and advanced its set's generation
    # past the wrap: 4 pair calls (one per set), or 8 single calls on set 0
    words = ws.view(torch.int32).cpu().numpy().view(np.uint32)
    want = {0: 2, 1: 2} if calls == "pair" else {0: 6}
    for s, g in want.items():
        assert words[_GRID_AT + s * _SET_WORDS + _TOP_AT + 4] == g, (calls, s)


@pytest.mark.parametrize("wait_polls", [0, 1])
def test_current_scaling_calls_of_many_sizes_share_a_workspace(F, orc, wait_polls):
    """Single and paired one-launch calls of different sizes (so different
    numbers of workgroup groups), and a transposed-copy call that takes the
    two-launch path, all in a row on one workspace: every call matches the
    oracle bit for bit (the grid-wide words one call leaves are valid for
    any next call, whatever its grid)."""
    ws = F.workspace(wait_polls=wait_polls)
    seq = [("one", (4096, 4096)), ("one", (256, 256)), ("pair", ((11008, 4096), (64, 64))),
           ("one", (2056, 8208)), ("t", (512, 768)), ("pair", ((256, 256), (4096, 4096))),
           ("one", (16, 16)), ("one", (11008, 4096))]
    for i, (kind, shp) in enumerate(seq):
        shapes = shp if kind == "pair" else (shp,)
        xs = [rand_bits(sh, 1100 + 10 * i + j, 1.5 if j == 0 else 0.03) for j, sh in enumerate(shapes)]
        dx = [dev_bf16(x) for x in xs]
        outs = [_current_outputs(sh) for sh in shapes]
        if kind == "pair":
            F.fp8_quantize_pair_current(dx[0], E4M3, *outs[0], dx[1], E4M3, *outs[1], workspace=ws)
        elif kind == "t":
            qT = empty_dev(shp[::-1], torch.uint8)
            F.fp8_quantize_tensor_current(dx[0], E4M3, outs[0][0], qT, *outs[0][1:], workspace=ws)
        else:
            F.fp8_quantize_tensor_current(dx[0], E4M3, outs[0][0], None, *outs[0][1:], workspace=ws)
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            _check_current(orc, xs[j], E4M3, *outs[j], label=f"call {i} {kind} {shapes[j]}")
        if kind == "t":
            assert np.array_equal(bytes8(qT), bytes8(outs[0][0]).T), f"call {i} qT"
