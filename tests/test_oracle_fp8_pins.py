"""Pins of the fp8 block-quantization oracle (oracle/mx_fp8.py) to the E4M3
format definition and to the MX scaling rule, by values fixed by the format,
an exhaustive nearest-value search, and the scaling identities."""
import numpy as np
import pytest

from oracle import mx_fp8 as mx


def test_e4m3_decode_fixed_values():
    d = mx.DECODE
    assert d[0x00] == 0 and d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x08] == 2.0 ** -6 and d[0x38] == 1.0 and d[0x40] == 2.0 and d[0x39] == 1.125
    assert d[0x7E] == 448.0 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0xB8] == -1.0 and d[0xFE] == -448.0 and d[0x80] == 0.0
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # increasing with the code
    assert np.array_equal(-d[0x80:0xFF], pos)           # sign bit mirrors


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if not np.isnan(mx.DECODE[c])], dtype=np.uint8)
    vals = mx.e4m3_decode(codes)
    assert np.array_equal(mx.e4m3_encode(vals), codes)


def _nearest_brute(x):
    """Independent nearest search over all finite codes: smallest distance,
    ties to the code with an even mantissa LSB, sign from x."""
    out = []
    for v in np.asarray(x, dtype=np.float64):
        best = None
        for c in range(0x7F):
            dist = abs(mx.DECODE[c] - abs(v))
            if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
                best = (dist, c)
        out.append(best[1] | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_ties_to_even_and_brute_force():
    pos = mx.DECODE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)   # midpoints exact in fp32
    enc = mx.e4m3_encode(mids)
    assert np.all(enc % 2 == 0)                           # every tie lands on an even code
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 400),
                        np.sign(rng.standard_normal(400)) * 2.0 ** rng.uniform(-12, 8.8, 400),
                        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500))])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(mx.e4m3_encode(x), _nearest_brute(x))


def test_mx_known_block():
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2] = 1.0, -0.5, 0.3
    c, e = mx.mx_quantize(x)
    assert e.tolist() == [119]                            # 1.0 <= 448 * 2^-8: X = -8
    assert c[0] == 0x78 and c[1] == 0xF0                  # 1.0 -> 256 = 2^8, -0.5 -> -128
    assert np.all(c[3:] == 0)
    assert abs(mx.mx_dequantize(c, e)[2] - 0.3) <= 0.3 * 2.0 ** -4


def test_mx_zero_and_subnormal_blocks():
    c, e = mx.mx_quantize(np.zeros((2, 64), dtype=np.float32))
    assert np.all(e == 0) and np.all(c == 0)
    tiny = np.full(32, 1e-40, dtype=np.float32)          # float32 subnormal amax
    c, e = mx.mx_quantize(tiny)
    assert e.tolist() == [0]
    assert np.all(mx.mx_dequantize(c, e) == mx.e4m3_decode(c) * np.float32(2.0 ** -127))


def test_mx_error_bound_and_top_binade():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * 2.0 ** rng.uniform(-20, 20, (64, 1))).astype(np.float32)
    x[3, 32:64] = 0
    c, e = mx.mx_quantize(x)
    xq = mx.mx_dequantize(c, e)
    scale = np.repeat(2.0 ** (e.astype(np.float64) - 127), 32, axis=1)
    # half an E4M3 step: 2^-4 relative for normals, 2^-10 * scale below 2^-6 * scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10)
    assert np.all(np.abs(xq - x) <= bound)
    # the largest element of every non-zero block lands in [224, 448]: the
    # scale is the smallest power of two that avoids clipping
    mag = np.abs(mx.e4m3_decode(c)).reshape(64, 4, 32).max(axis=2)
    nz = np.abs(x).reshape(64, 4, 32).max(axis=2) > 0
    assert np.all(mag[nz] >= 224) and np.all(mag[nz] <= 448) and np.all(mag[~nz] == 0)


def test_mx_power_of_two_invariance_and_axis():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    c1, e1 = mx.mx_quantize(x)
    c2, e2 = mx.mx_quantize(x * np.float32(2.0 ** 5))
    assert np.array_equal(c1, c2) and np.array_equal(e2.astype(int), e1.astype(int) + 5)
    # blocking along another axis is the transpose of blocking the transpose
    y = rng.standard_normal((64, 8)).astype(np.float32)
    ca, ea = mx.mx_quantize(y, axis=0)
    cb, eb = mx.mx_quantize(y.T, axis=-1)
    assert np.array_equal(ca, cb.T) and np.array_equal(ea, eb.T)
    assert np.array_equal(mx.mx_dequantize(ca, ea, axis=0), mx.mx_dequantize(cb, eb).T)


def test_mx_scale_choice_at_the_range_edge():
    """448 * 2^k fits with X = k; anything above needs X = k + 1."""
    for amax, want_E, want_code in ((448.0, 127, 0x7E), (449.0, 128, 0x76), (511.0, 128, 0x78),
                                    (224.0, 126, 0x7E), (0.875, 118, 0x7E), (1.75, 119, 0x7E)):
        x = np.zeros(32, dtype=np.float32)
        x[0] = amax
        c, e = mx.mx_quantize(x)
        assert e.tolist() == [want_E] and c[0] == want_code, amax
        assert abs(mx.mx_dequantize(c, e)[0] - amax) <= amax * 2.0 ** -4


def test_planted_encoder_mistake_is_caught():
    """Round half away from zero in place of ties-to-even disagrees with the
    brute-force pin on midpoints."""
    pos = mx.DECODE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    away = np.searchsorted(pos, mids.astype(np.float64), side="left").astype(np.uint8)
    assert not np.array_equal(away, _nearest_brute(mids))
