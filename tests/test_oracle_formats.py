"""Pins of the oracle's FP8 E4M3 / FP16 rounding against independent implementations
(torch's float8_e4m3fn cast, numpy's float16) and against the rounding definitions."""

import numpy as np
import pytest
import torch

from oracle import formats


def test_e4m3_table_matches_format_definition_limits():
    v = formats.E4M3_DECODE
    finite = v[~np.isnan(v)]
    assert np.isnan(v).sum() == 2                      # 0x7F and 0xFF
    assert finite.max() == 448.0 and finite.min() == -448.0
    pos = np.unique(finite[finite > 0])
    assert pos[0] == 2.0 ** -9                         # smallest subnormal
    assert 2.0 ** -6 in pos and 2.0 ** -6 - 2.0 ** -9 in pos
    assert len(pos) == 126


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = formats.E4M3_DECODE
    same = (tv == ov) | (np.isnan(tv) & np.isnan(ov))
    assert same.all()


def test_e4m3_rne_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 200000)),
        formats.E4M3_DECODE[:0x7F],                                    # exact values
        (formats.E4M3_DECODE[1:0x7F] + formats.E4M3_DECODE[:0x7E]) / 2,  # exact ties
        [0.0, 448.0],
    ])
    x = x[x <= 448.0]
    ours, codes = formats.e4m3_rne(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn)
    assert np.array_equal(ours, theirs.to(torch.float64).numpy())
    assert np.array_equal(codes, theirs.view(torch.uint8).numpy())


def test_e4m3_ru_is_smallest_value_not_below():
    rng = np.random.default_rng(8)
    x = np.concatenate([np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 50000)),
                        formats.E4M3_DECODE[:0x7F]])
    vals, codes = formats.e4m3_ru(x)
    assert np.all(vals >= x)
    below = formats.E4M3_DECODE[np.maximum(codes.astype(int) - 1, 0)]
    assert np.all((codes == 0) | (below < x))
    exact = np.isin(x, formats.E4M3_DECODE)
    assert np.array_equal(vals[exact], x[exact])


def test_fp16_rd_against_numpy_nextafter():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000) * np.exp(rng.uniform(-20, 10, 100000)),
                        np.float16(rng.standard_normal(1000)).astype(np.float64),
                        [0.0, -0.0, 65504.0, -65504.0, 2.0 ** -24, -(2.0 ** -24)]])
    x = x[np.abs(x) <= 65504.0]
    vals, bits = formats.fp16_rd(x)
    h = x.astype(np.float16)                     # round to nearest
    over = h.astype(np.float64) > x
    with np.errstate(over="ignore"):
        down = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    expect = np.where(over, down, h.astype(np.float64))
    assert np.array_equal(vals, expect)
    assert np.all(vals <= x)
    assert np.array_equal(formats.fp16_value(bits), vals)


def test_fp16_table_limits():
    f = formats.FP16_DECODE
    assert np.nanmax(f) == 65504.0
    assert np.isnan(f).sum() == 2 * 1024  # exponent 31 (inf and NaN patterns) is excluded
    assert formats.fp16_value(np.uint16(1)) == 2.0 ** -24


@pytest.mark.parametrize("bad", [-1.0, 449.0, float("nan")])
def test_e4m3_rejects_out_of_range(bad):
    with pytest.raises(ValueError):
        formats.e4m3_rne([bad])
    with pytest.raises(ValueError):
        formats.e4m3_ru([bad])
