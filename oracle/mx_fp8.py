"""fp8 (OCP E4M3) block quantization with shared power-of-two scales.
TEST INFRASTRUCTURE, like the rest of this package.

The low-precision variant of the method quantizes its inputs block by block,
each block with its own scale (zzszmyf.github.io notes "FlashAttention
原理是什么", section 10 item ③ and section 12.2: per-block scales are more
stable than one scale per tensor).  The pages fix neither the block shape nor
the scale format; the reading taken here is the microscaling (MX) layout that
gfx950's matrix cores consume directly: blocks of 32 consecutive elements
along the contracted dimension share one scale 2^X stored as an E8M0 byte
(E = X + 127), with X the smallest integer that brings the block's largest
magnitude within the E4M3 range, so no element is clipped.  For one block
x_0..x_31 (float32), with amax = max |x_i| = m * 2^f (1 <= m < 2):

    X    = f - 8 if m <= 1.75 else f - 7     (smallest X with amax <= 448 * 2^X)
    E    = clamp(X + 127, 0, 254)             (zero or subnormal amax: E = 0)
    c_i  = E4M3_rne(clamp(x_i * 2^(127 - E), -448, 448))

f and m are read from the float32 bit pattern (exponent field, and the
mantissa field compared with that of 1.75), so the choice of X is exact;
every product is a power-of-two scaling and exact; the clamp never binds
for finite inputs; E4M3_rne is the nearest E4M3 value with ties to the even
code.  The dequantized value is decode(c_i) * 2^(E - 127), exact in float32.

E4M3 (OCP 8-bit floating point, E4M3 variant): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
m * 2^-9; the all-ones code S.1111.111 is NaN and there is no infinity, so
the largest finite value is 1.75 * 2^8 = 448.

Incoherent processing (notes page, section 10 item ③ and section 12.2):
before block quantization, Q and K rows can be rotated by an orthogonal
transform that spreads outlier channels over all head dims; since
(Q R)(K R)^T = Q R R^T K^T, an orthogonal R leaves the scores unchanged.  The
reading taken here: R = diag(s) H_d with H_d the Sylvester-Hadamard matrix of
order d (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), entries +-1 and
H H^T = d I, and s a sign per head dim (an input, drawn by the caller).  It
is not normalised, so (Q R)(K R)^T = d Q K^T and the attention over rotated
inputs takes scale / d, an exact power-of-two change.  The rotated row is
computed in float64 (the products by +-1 and the sums are exact for
bf16-valued rows whose magnitudes span fewer than 2^38) and rounded once to
float32, an exact zero taken as +0 (its sign would otherwise depend on the
order of the sums); the MX quantization above then applies unchanged.

Functions
  e4m3_decode(codes)              -> float32 values
  e4m3_encode(x)                  -> uint8 codes, x already within [-448, 448]
  mx_quantize(x, axis=-1)         -> (codes uint8, scales uint8), blocks of 32
                                     consecutive elements along `axis`
  mx_dequantize(codes, scales, axis=-1) -> float32
  hadamard(d)                     -> float64 [d, d] Sylvester-Hadamard matrix
  rotate_rows(x, signs=None)      -> float32 rows of x diag(signs) H_d
"""
import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def _decode_one(c):
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7e, increasing in value
_POS = DECODE[:0x7F]


def e4m3_decode(codes):
    return DECODE[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x):
    """Nearest E4M3 code of each float32 value in [-448, 448]; ties go to the
    even code (mantissa LSB 0).  -0.0 encodes as 0x80."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode expects finite values within +-448")
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return code | sign


def _blocks_last(x, axis):
    x = np.moveaxis(np.asarray(x, dtype=np.float32), axis, -1)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("the blocked axis must be a multiple of 32")
    return x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))


def mx_quantize(x, axis=-1):
    """Codes (same shape as x) and E8M0 scales (the blocked axis divided by
    32) of the MX E4M3 quantization of float32 x."""
    xb = _blocks_last(x, axis)
    amax = np.abs(xb).max(axis=-1)
    bits = amax.view(np.uint32).astype(np.int64)
    field = (bits >> 23) & 0xFF
    over = ((bits & 0x7FFFFF) > 0x600000).astype(np.int64)   # mantissa above 1.75
    E = np.where(field == 0, 0, np.clip(field - 8 + over, 0, 254))
    scaled = np.ldexp(xb, (127 - E)[..., None].astype(np.int32)).astype(np.float32)
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(scaled)
    codes = codes.reshape(codes.shape[:-2] + (-1,))
    return np.moveaxis(codes, -1, axis), np.moveaxis(E.astype(np.uint8), -1, axis)


def mx_dequantize(codes, scales, axis=-1):
    """float32 values decode(c) * 2^(E - 127)."""
    cb = _blocks_last(e4m3_decode(codes), axis)
    E = np.moveaxis(np.asarray(scales, dtype=np.int64), axis, -1)
    out = np.ldexp(cb, (E - 127)[..., None].astype(np.int32)).astype(np.float32)
    out = out.reshape(out.shape[:-2] + (-1,))
    return np.moveaxis(out, -1, axis)


def hadamard(d):
    """The Sylvester-Hadamard matrix of order d (a power of two), float64."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_rows(x, signs=None):
    """x diag(signs) H_d along the last axis (d = x.shape[-1]), in float64,
    rounded once to float32.  signs: d values, an entry < 0 flips that head
    dim; None flips none."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    d = x.shape[-1]
    if signs is not None:
        x = x * np.where(np.asarray(signs) < 0, -1.0, 1.0)
    # an exact zero is +0, whichever signed zeros or terms produced it
    return (x @ hadamard(d) + 0.0).astype(np.float32)
