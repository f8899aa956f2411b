"""Pins for the oracle INT4 quantizer (CPU only).

Each check comes from something other than the oracle itself: hand-worked
groups (tests/golden/quant_group.txt), closed forms of constructed inputs,
error bounds, and the degenerate constant group.
"""
import os

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_group.txt")


def _golden_cases():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        cur[key] = val.split()
        if key == "codes":
            cases.append(cur)
            cur = {}
    return cases


@pytest.mark.parametrize("case", range(5))
def test_golden_groups(case):
    c = _golden_cases()[case]
    x = np.array([np.float32(v) for v in c["x"]], dtype=np.float32)
    codes, s, z = quant.quantize_groups(x[None, :], 32)
    assert float(s[0, 0]) == float(c["scale"][0])
    assert float(z[0, 0]) == float(c["zero"][0])
    assert codes[0].tolist() == [int(v) for v in c["codes"]]


def _exact_group(rng, c):
    """x = z + c * s with fp16 s, z, exact in float32, for codes c (0 and 15 present)."""
    while True:
        s = np.float16(rng.uniform(0.01, 2.0))
        z = np.float16(rng.uniform(-4.0, 4.0))
        x64 = float(z) + c.astype(np.float64) * float(s)
        x32 = x64.astype(np.float32)
        if np.array_equal(x32.astype(np.float64), x64):
            # 15 s must also be exact, so that (max - min) / 15 == s in fp32
            if np.float32(np.float32(15.0 * float(s)) / np.float32(15)) == np.float32(s):
                return x32, s, z


def test_closed_form_every_code():
    rng = np.random.default_rng(5)
    for _ in range(200):
        c = np.concatenate([np.arange(16), rng.integers(0, 16, 16)])
        rng.shuffle(c)
        x, s, z = _exact_group(rng, c)
        codes, s16, z16 = quant.quantize_groups(x[None], 32)
        assert s16[0, 0] == s and z16[0, 0] == z
        assert np.array_equal(codes[0], c)


def test_half_way_ties_round_to_even():
    rng = np.random.default_rng(6)
    hits = 0
    for _ in range(300):
        c = np.concatenate([[0, 15], rng.integers(0, 15, 30)])
        x, s, z = _exact_group(rng, c.astype(np.int64))
        # move elements 2.. to the half-way point c + 1/2 where exact
        xt = x.astype(np.float64).copy()
        want = c.copy()
        for i in range(2, 32):
            v = float(z) + (c[i] + 0.5) * float(s)
            if np.float64(np.float32(v)) == v and \
               np.float32(np.float32(v) - np.float32(z)) == np.float32(v - float(z)):
                xt[i] = v
                want[i] = c[i] if c[i] % 2 == 0 else c[i] + 1
                hits += 1
        codes, _, _ = quant.quantize_groups(xt.astype(np.float32)[None], 32)
        assert np.array_equal(codes[0], want)
    assert hits > 1000


def test_error_bound_and_range():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((4096, 128)) * rng.uniform(0.1, 20, (4096, 1))).astype(np.float32)
    codes, s, z = quant.quantize_groups(x, 32)
    assert codes.min() >= 0 and codes.max() <= 15
    xh = quant.dequantize_groups(codes, s, z, 32).reshape(4096, 4, 32)
    g = x.astype(np.float64).reshape(4096, 4, 32)
    sf = s.astype(np.float64)[..., None]
    zf = z.astype(np.float64)[..., None]
    mn = g.min(-1, keepdims=True)
    mx = g.max(-1, keepdims=True)
    delta = np.maximum(0, np.maximum(zf - mn, mx - (zf + 15 * sf)))
    err = np.abs(g - xh)
    assert np.all(err <= sf / 2 * (1 + 1e-5) + delta + 1e-7)
    # the reconstruction is much better than the group range for every group
    assert np.all(err.max(-1) <= (mx - mn)[..., 0] / 15.0 + 1e-6)


def test_constant_group():
    x = np.full((3, 64), 2.75, dtype=np.float32)
    x[1, 32:] = -1.5
    codes, s, z = quant.quantize_groups(x, 32)
    assert np.all(codes == 0) and np.all(s == 0)
    assert z[0].tolist() == [2.75, 2.75] and z[1].tolist() == [2.75, -1.5]
    xh = quant.dequantize_groups(codes, s, z, 32)
    assert np.array_equal(xh, x.astype(np.float64))


def test_packing_nibble_order():
    codes = np.array([[1, 2, 15, 0, 7, 8]], dtype=np.uint8)
    packed = quant.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x0F, 0x87]]
    assert np.array_equal(quant.unpack_nibbles(packed), codes)


def test_storage_round_trip():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((17, 64)).astype(np.float32)
    packed, sz = quant.quantize_rows(x, 32)
    assert packed.shape == (17, 32) and sz.shape == (17, 2, 2) and sz.dtype == np.uint16
    codes, s, z = quant.quantize_groups(x, 32)
    s2, z2 = quant.split_scale_zero(sz)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(z2.view(np.uint16), z.view(np.uint16))
    assert np.array_equal(quant.dequantize_rows(packed, sz, 32),
                          quant.dequantize_groups(codes, s, z, 32))


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        quant.quantize_groups(np.array([[np.nan] * 32], dtype=np.float32))
    with pytest.raises(ValueError):
        quant.quantize_groups(np.array([[1e6] * 32], dtype=np.float32))
    with pytest.raises(ValueError):
        quant.quantize_groups(np.array([[0.1] * 32], dtype=np.float64))  # not exact in fp32


def test_signed_zero_is_canonical():
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, ::2] = -0.0
    x[1, 5] = 0.5
    x[1, 6] = -0.0
    codes, s, z = quant.quantize_groups(x, 32)
    assert s.view(np.uint16)[0, 0] == 0 and z.view(np.uint16).tolist() == [[0], [0]]
