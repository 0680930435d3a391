"""Oracle pins against the figures the pages print (fixtures in tests/golden/).

* The FP8 bit splits of the FP8 quantisation training guide (section "format
  choice: E4M3 and E5M2") fix each format's code structure: 2^mantissa values
  per binade, bias 2^(exponent-1) - 1, the smallest normal and subnormal, and,
  under the OCP readings (E4M3 without infinities, its all-ones code NaN; E5M2
  with IEEE-style infinities), the largest finite value.  The oracle's decode
  table must show exactly that structure.
* The block shapes of the guide's "blockwise scaling" and "MXFP8 scaling"
  sections fix which elements share a scale: an outlier planted anywhere must
  change the scale of exactly one block, the one of the printed extent that
  holds it, and the scale grids must have the printed block counts.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def _formats():
    return {r[0]: (int(r[1]), int(r[2]), int(r[3])) for r in _rows("fp8_formats.txt")}


def _blocks():
    return [dict(recipe=r[0], role=r[1], br=int(r[2]), bc=int(r[3]), elem=r[4], scale=r[5])
            for r in _rows("block_geometry.txt")]


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_decode_table_has_the_printed_bit_split(orc, name):
    sign, ebits, mbits = _formats()[name]
    assert sign == 1
    fmt = orc.E4M3 if name == "E4M3" else orc.E5M2
    tab = orc.decode_table(fmt)
    bias = 2 ** (ebits - 1) - 1
    # every code, decoded from its fields under the printed split
    for c in range(256):
        s = -1 if c >> (ebits + mbits) else 1
        e = (c >> mbits) & ((1 << ebits) - 1)
        m = c & ((1 << mbits) - 1)
        top = e == (1 << ebits) - 1
        if name == "E4M3" and top and m == (1 << mbits) - 1:
            assert np.isnan(tab[c]), c          # the only NaN pattern (no inf)
            continue
        if name == "E5M2" and top:
            assert np.isinf(tab[c]) if m == 0 else np.isnan(tab[c]), c
            continue
        if e == 0:
            v = Fraction(m, 2 ** mbits) * Fraction(2) ** (1 - bias)
        else:
            v = (1 + Fraction(m, 2 ** mbits)) * Fraction(2) ** (e - bias)
        assert Fraction(tab[c]) == s * v, (name, c)
    fin = tab[np.isfinite(tab)]
    assert Fraction(fin[fin > 0].min()) == Fraction(2) ** (1 - bias - mbits)
    assert Fraction(fin[fin >= 2.0 ** (1 - bias)].min()) == Fraction(2) ** (1 - bias)
    top_e = (2 ** ebits - 1) if name == "E4M3" else (2 ** ebits - 2)
    top_m = (2 ** mbits - 2) if name == "E4M3" else (2 ** mbits - 1)
    vmax = (1 + Fraction(top_m, 2 ** mbits)) * Fraction(2) ** (top_e - bias)
    assert Fraction(fin.max()) == vmax
    assert float(vmax) == orc.FMAX[fmt]        # 448 and 57344
    # 2^mbits values per binade: consecutive positive normals step by 2^-mbits
    for e in range(1, top_e):
        binade = tab[(e << mbits):((e + 1) << mbits)]
        steps = np.diff(binade) / (2.0 ** (e - bias))
        assert np.all(steps == 2.0 ** -mbits)


def test_e8m0_scale_is_a_bare_power_of_two(orc):
    sign, ebits, mbits = _formats()["E8M0"]
    assert (sign, ebits, mbits) == (0, 8, 0)
    rng = np.random.Generator(np.random.PCG64(7))
    x = orc.f64_to_bf16(rng.standard_normal((4, 256)) * np.exp(rng.uniform(-20, 20, (4, 1))))
    q, e = orc.quantize_mx(x, orc.E4M3)
    xs = orc.bf16_to_f32(x).astype(np.float64)
    tab = orc.decode_table(orc.E4M3)
    deq = tab[q] * np.repeat(np.exp2(e.astype(np.float64) - (2 ** (ebits - 1) - 1)), 32, axis=1)
    # one power-of-two multiplier per block reconstructs x to E4M3 precision
    assert np.all(np.abs(deq - xs) <= 2.0 ** -4 * np.abs(xs) + 1e-300 +
                  np.repeat(np.exp2(e.astype(np.float64) - 127 - 9), 32, axis=1))


def _plant_and_diff(orc, quant, shape, r, c, rng):
    base = orc.f64_to_bf16(rng.standard_normal(shape))
    s0 = quant(base)
    x = base.copy()
    x[r, c] = orc.f64_to_bf16(np.array([1e4]))[0]
    s1 = quant(x)
    return np.argwhere(s0 != s1)


@pytest.mark.parametrize("row", [0, 1, 2], ids=["activation", "gradient", "weight"])
def test_blockwise_scale_extent_is_the_printed_one(orc, row):
    b = _blocks()[row]
    assert b["recipe"] == "blockwise" and b["elem"] == "E4M3"
    R, C = 256, 384
    rng = np.random.Generator(np.random.PCG64(11 + row))

    def quant(x):
        return orc.quantize_block(x, orc.E4M3, b["br"], b["bc"])[1]

    assert quant(orc.f64_to_bf16(np.ones((R, C)))).shape == (R // b["br"], C // b["bc"])
    for r, c in [(0, 0), (127, 127), (128, 128), (200, 300), (255, 383)]:
        changed = _plant_and_diff(orc, quant, (R, C), r, c, rng)
        assert changed.tolist() == [[r // b["br"], c // b["bc"]]]


def test_mx_scale_extent_is_the_printed_one(orc):
    b = _blocks()[3]
    assert b["recipe"] == "mxfp8" and b["scale"] == "E8M0"
    R, C = 8, 256
    rng = np.random.Generator(np.random.PCG64(17))

    def quant(x):
        return orc.quantize_mx(x, orc.E4M3)[1]

    assert quant(orc.f64_to_bf16(np.ones((R, C)))).shape == (R // b["br"], C // b["bc"])
    for r, c in [(0, 0), (0, 31), (0, 32), (3, 100), (7, 255)]:
        changed = _plant_and_diff(orc, quant, (R, C), r, c, rng)
        assert changed.tolist() == [[r // b["br"], c // b["bc"]]]
