"""Pins of the fp8 block-quantization oracle (oracle/mx_fp8.py) to the E4M3
format definition and to the MX scaling rule, by values fixed by the format,
an exhaustive nearest-value search, and the scaling identities."""
import numpy as np
import pytest

from io_aware_softmax_fwd_amd import workloads as W
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


# ------------------------------------------------- incoherent processing
def test_hadamard_small_orders_written_out():
    assert np.array_equal(mx.hadamard(1), [[1.0]])
    assert np.array_equal(mx.hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(mx.hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("d", [64, 128])
def test_hadamard_closed_form_and_orthogonality(d):
    """Entry (i, j) of the Sylvester construction is (-1)^popcount(i & j),
    and H H^T = d I."""
    h = mx.hadamard(d)
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(h, np.where(parity == 1, -1.0, 1.0))
    assert np.array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_preserves_scores_up_to_d(d):
    """(q R)(k R)^T = d q k^T with R = diag(s) H: exact in float64 for
    bf16-valued rows, so the float32 rounding of the rotated rows is the
    only difference; rotating back (R^T / d) recovers the row."""
    rng = np.random.default_rng(d)
    bf = lambda a: W.bf16_bits_to_f32(W.bf16_bits_rne(a.astype(np.float32)))
    q = bf(rng.standard_normal((20, d)))
    k = bf(rng.standard_normal((30, d)))
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    qr, kr = mx.rotate_rows(q, s), mx.rotate_rows(k, s)
    exact = d * (q.astype(np.float64) @ k.astype(np.float64).T)
    got = qr.astype(np.float64) @ kr.astype(np.float64).T
    # each rotated entry carries at most half an fp32 ulp of relative error
    bound = 2.0 ** -23 * (np.abs(qr).astype(np.float64) @ np.abs(kr).astype(np.float64).T)
    assert np.all(np.abs(got - exact) <= bound)
    back = (qr.astype(np.float64) @ mx.hadamard(d).T / d) * np.where(s < 0, -1.0, 1.0)
    assert np.allclose(back, q, rtol=0, atol=2.0 ** -20 * np.abs(q).max())
    # without signs the first column of H is all ones: entry 0 is the row sum
    r0 = mx.rotate_rows(q)
    assert np.array_equal(r0[:, 0], q.astype(np.float64).sum(axis=1).astype(np.float32))


def test_rotation_spreads_an_outlier_channel():
    """A row that is zero except one head dim becomes a row of equal
    magnitudes: the outlier is spread over all d dims (so one E4M3 block
    scale no longer has to cover it alone)."""
    d = 128
    x = np.zeros((1, d), dtype=np.float32)
    x[0, 37] = 50.0
    r = mx.rotate_rows(x)
    assert np.array_equal(np.abs(r), np.full((1, d), 50.0, dtype=np.float32))


def test_rotation_of_signed_zeros_is_plus_zero():
    """A zero row, with any signs, rotates to +0 in every dim (code 0x00)."""
    x = np.zeros((2, 64), dtype=np.float32)
    x[1] = -0.0
    s = np.where(np.arange(64) % 3 == 0, -1, 1).astype(np.int8)
    r = mx.rotate_rows(x, s)
    assert np.all(r == 0) and not np.any(np.signbit(r))
    c, e = mx.mx_quantize(r)
    assert np.all(c == 0) and np.all(e == 0)
