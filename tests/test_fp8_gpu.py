"""Parity of the fp8 path: the MX block quantizers (plain and rotated) bit
for bit against the oracle's quantization, and the fp8 attention forward
against the oracle's attention of the dequantized inputs.

Tolerances of the attention, per element, in three parts:
 * Hard pin (no model): inputs whose probabilities are all powers of two,
   exact in E4M3, leave only the bf16 rounding of O and the accumulation
   term below; there O must be within 4e-3 max|O| and LSE within 1e-3.
 * Statistical bound for P rounding (a model, not a worst case): the kernel
   rounds the probabilities P to E4M3 before the product with V and sums the
   same rounded values for the denominator.  Rounding P_j changes weight
   w_j = P_j / l by at most e_j = max(delta * w_j, 2^-10 / l), delta = 2^-4
   (half an E4M3 step, relative, for normal values; 2^-10 absolute below
   2^-6, in units where the row's largest P is at least 1, so l >= 1).
   Modelling these errors as independent and uniform across keys, the
   error of O_c has standard deviation
       sigma_c = sqrt(sum_j e_j^2 / 3 * (v_jc - O_c)^2)
   and the test allows 8 sigma_c (LSE: 8 sqrt(sum_j e_j^2 / 3)), plus half
   a bf16 step of O (2^-9 |O|, doubled) and, for LSE, 1e-3.
 * Accumulation (a stated assumption): AMD documents no error bound for the
   internal accumulation of v_mfma_scale_f32_32x32x64_f8f6f4.  The tests
   assume that it adds at most 3e-4 max_j |v_jc| to O_c (an fp32 accumulation
   would add about 1e-6; the allowance covers a reduced-precision internal
   sum of the 64 products of each instruction).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import mx_fp8 as mx
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

DELTA = 2.0 ** -4


def _bf(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _perm():
    """Key (inside a 64-key tile) held by position p = 32h + j of a tile row."""
    return np.array([32 * (j // 16) + (j % 4) + 8 * ((j % 16) // 4) + 4 * h
                     for h in (0, 1) for j in range(32)])


def _v_logical(v8t, vs, BH, N, d):
    """GPU V layout -> codes [BH, T*64, d] and scales [BH, 2T, d] in key order."""
    T = (N + 63) // 64
    tiles = v8t.reshape(BH, T, d, 64).transpose(0, 1, 3, 2)        # [BH, T, position, d]
    codes = np.zeros((BH, T, 64, d), dtype=np.uint8)
    codes[:, :, _perm(), :] = tiles
    scales = vs.reshape(BH, T, 2, 32, d // 32).transpose(0, 1, 2, 4, 3).reshape(BH, 2 * T, d)
    return codes.reshape(BH, T * 64, d), scales


def _oracle_quant(q, k, v):
    """Oracle MX quantization of q, k, v ([B,H,N,d] float32): codes, scales and
    the dequantized float32 inputs (V padded to whole 64-key tiles)."""
    B, H, N, d = q.shape
    T = (N + 63) // 64
    qc, qs = mx.mx_quantize(q, axis=-1)
    kc, ks = mx.mx_quantize(k, axis=-1)
    vp = np.zeros((B * H, T * 64, d), dtype=np.float32)
    vp[:, :N] = v.reshape(B * H, N, d)
    vc, vsc = mx.mx_quantize(vp, axis=-2)
    deq = (mx.mx_dequantize(qc, qs), mx.mx_dequantize(kc, ks),
           mx.mx_dequantize(vc, vsc, axis=-2)[:, :N].reshape(B, H, N, d))
    return (qc, qs, kc, ks, vc, vsc), deq


def _gpu_quant(q, k, v):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    q8, qs = fa.quantize_qk_fp8(qd)
    k8, ks = fa.quantize_qk_fp8(kd)
    v8t, vs = fa.quantize_v_fp8(vd)
    torch.cuda.synchronize()
    return q8, qs, k8, ks, v8t, vs


def _special_values(shape, seed):
    """bf16 values spanning the scale rule's corner cases: block maxima just
    at and above 1.75 * 2^k, zero blocks, bf16 subnormals, huge and tiny
    rows, negative zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= (2.0 ** rng.integers(-40, 40, size=shape[:-1] + (1,))).astype(np.float32)
    flat = x.reshape(-1, shape[-1])
    n = flat.shape[0]
    flat[0::7, :32] = 0.0
    flat[1::7, :32] = np.float32(1.75) * np.sign(flat[1::7, :32] + 0.5)
    flat[2::7, 5] = np.float32(1.7578125) * 8             # first bf16 above 1.75, scaled
    flat[3::7, :] *= np.float32(1e-38)                    # float32/bf16 subnormals
    flat[4::7, 3] = -0.0
    flat[5::7, :] = np.float32(448.0)
    x = flat.reshape(shape)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


@pytest.mark.parametrize("N,d", [(100, 64), (300, 128), (64, 128), (1, 64)])
def test_quantizers_bit_exact(N, d):
    torch_or_skip()
    B, H = 1, 3
    note("fp8 quantizers N=%d d=%d" % (N, d))
    q = _special_values((B, H, N, d), 1 + N)
    k = _bf((B, H, N, d), 2 + N, 3.0)
    v = _special_values((B, H, N, d), 3 + N)
    g = [t.cpu().numpy() for t in _gpu_quant(q, k, v)]
    (qc, qs, kc, ks, vc, vsc), _ = _oracle_quant(q, k, v)
    assert np.array_equal(g[0], qc) and np.array_equal(g[1], qs)
    assert np.array_equal(g[2], kc) and np.array_equal(g[3], ks)
    gvc, gvs = _v_logical(g[4], g[5], B * H, N, d)
    assert np.array_equal(gvs, vsc)
    assert np.array_equal(gvc, vc)


def _bounds(qd, kd, vd, scale, causal, rows, O_ref):
    """Per-element O bound and per-row LSE bound of the docstring for the
    listed flat rows (float64 numpy on the dequantized inputs)."""
    B, H, N, d = qd.shape
    ob = np.empty((len(rows), d))
    lb = np.empty(len(rows))
    for t, r in enumerate(rows):
        bh, i = divmod(int(r), N)
        b, h = divmod(bh, H)
        nk = i + 1 if causal else N
        s = scale * (kd[b, h, :nk].astype(np.float64) @ qd[b, h, i].astype(np.float64))
        p = np.exp(s - s.max())
        l = p.sum()
        w = p / l
        e = np.maximum(DELTA * w, 2.0 ** -10 / l)
        vv = vd[b, h, :nk].astype(np.float64)
        sig = np.sqrt((e[:, None] ** 2 / 3 * (vv - O_ref[t][None, :]) ** 2).sum(axis=0))
        ob[t] = 8 * sig + 2.0 ** -8 * np.abs(O_ref[t]) + 3e-4 * np.abs(vv).max(axis=0)
        lb[t] = 8 * math.sqrt((e ** 2).sum() / 3) + 1e-3
    return ob, lb


def _run_fp8(q8, qs, k8, ks, v8t, vs, scale, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    o, lse = fa.fwd_fp8(q8, qs, k8, ks, v8t, vs, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check_rows(O, L, deq, scale, causal, rows, what):
    qd, kd, vd = deq
    B, H, N, d = qd.shape
    O_ref, L_ref = oracle.attention_c(qd, kd, vd, scale, causal, rows=rows)
    Og = O.reshape(-1, d)[rows]
    Lg = L.reshape(-1)[rows]
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Lg)), what + ": non-finite"
    ob, lb = _bounds(qd, kd, vd, scale, causal, rows, O_ref)
    eo = np.abs(Og - O_ref)
    el = np.abs(Lg - L_ref)
    note("%s: max|dO|=%.3e (max|O| %.3e), worst dO/bound=%.3f, max|dLSE|=%.3e, worst dLSE/bound=%.3f"
         % (what, eo.max(), np.abs(O_ref).max(), (eo / ob).max(), el.max(), (el / lb).max()))
    assert np.all(eo <= ob), what + ": O outside the derived bound"
    assert np.all(el <= lb), what + ": LSE outside the derived bound"


# At d = 64 the kernel walks the key tiles three at a time (the product with
# V of tile j - 1, the softmax of tile j and the scores of tile j + 1 in one
# step), with separate code for one or two tiles in all, for an odd or even
# number of unmasked tiles, and for a tail of one or two tiles: the d = 64
# shapes below take each of these.  Calls of at most 192 workgroups of 128
# rows with at least 8 key tiles (N > 448) run the small-grid kernel instead
# (32-row workgroups whose waves split the keys): the shapes with N >= 449
# and few heads take it, (1, 48, 1000, 64, True) the walk above.
@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 300, 64, True), (2, 2, 257, 128, False),
                                             (1, 1, 1000, 128, True), (1, 2, 64, 64, False),
                                             (1, 1, 1, 128, True),
                                             (1, 1, 1, 64, False), (1, 2, 40, 64, True),
                                             (1, 2, 65, 64, True), (1, 1, 128, 64, False),
                                             (1, 3, 129, 64, False), (2, 1, 192, 64, True),
                                             (1, 1, 257, 64, True), (1, 2, 384, 64, False),
                                             (1, 1, 449, 64, True), (2, 2, 520, 128, False),
                                             (1, 3, 700, 64, False), (2, 1, 513, 64, True),
                                             (1, 48, 1000, 64, True)])
def test_fp8_random_within_derived_bound(B, H, N, d, causal):
    torch_or_skip()
    case = "fp8 random B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal)
    note(case)
    q, k, v = (_bf((B, H, N, d), 40 + N + d + t) for t in range(3))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = _run_fp8(*_gpu_quant(q, k, v), scale, causal)
    _, deq = _oracle_quant(q, k, v)
    _check_rows(O, L, deq, scale, causal, np.arange(B * H * N), case)


@pytest.mark.parametrize("N,d,causal", [(300, 64, True), (257, 128, False), (700, 128, True)])
def test_fp8_exact_probabilities_tight(N, d, causal):
    """Scores are small integers and scale = ln 2, so every probability the
    kernel forms is a power of two between 2^-9 and 2^8: exact in E4M3."""
    torch_or_skip()
    case = "fp8 exact-P N=%d d=%d causal=%d" % (N, d, causal)
    note(case)
    rng = np.random.default_rng(N + d)
    B, H = 1, 2
    q = np.zeros((B, H, N, d), dtype=np.float32)
    k = np.zeros((B, H, N, d), dtype=np.float32)
    idx = np.arange(N)
    for h in range(H):
        q[0, h, idx, rng.integers(0, 4, N)] = rng.integers(0, 4, N)
        k[0, h, idx, rng.integers(0, 4, N)] = rng.integers(0, 4, N)
    v = _bf((B, H, N, d), 7 + N)
    scale = float(np.float32(math.log(2.0)))
    O, L = _run_fp8(*_gpu_quant(q, k, v), scale, causal)
    _, deq = _oracle_quant(q, k, v)
    assert np.array_equal(deq[0], q) and np.array_equal(deq[1], k)   # integers survive exactly
    O_ref, L_ref = oracle.attention_c(*deq, scale, causal)
    eo, el = np.abs(O - O_ref).max(), np.abs(L - L_ref).max()
    note("%s: max|dO|=%.3e (bound %.3e)  max|dLSE|=%.3e (bound 1e-3)" % (case, eo, 4e-3 * np.abs(O_ref).max(), el))
    assert eo <= 4e-3 * np.abs(O_ref).max() and el <= 1e-3


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_workload_shapes(cfg):
    """The forward workloads' shapes and input recipes (C4 with its
    amplified rows) on sampled rows, against the derived bound."""
    torch_or_skip()
    w = W.WORKLOADS[cfg]
    if w.dtype != "bf16":
        pytest.skip("bf16 workloads only")
    note("fp8 workload C%d: %s" % (cfg, w.describe()))
    x = W.make_inputs(w)
    O, L = _run_fp8(*_gpu_quant(x["q"], x["k"], x["v"]), w.scale, w.causal)
    _, deq = _oracle_quant(x["q"], x["k"], x["v"])
    rows = W.sample_rows(w, 256, seed=cfg + 50)
    _check_rows(O, L, deq, w.scale, w.causal, rows, "C%d" % cfg)


@pytest.mark.parametrize("H", [2, 64])   # the small-grid kernel, the 128-row kernel
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_offset_moves(d, causal, H):
    """Keys whose score against every query sits far above all earlier keys
    (by 69, 173 and 231 log2 units; one on the ragged last tile) and one far
    below: the row max passes the exponent offset by far more than the
    8-unit headroom on those tiles, so the offset moves there mid-row and
    the accumulators are rescaled before the probabilities are rounded to
    E4M3."""
    torch_or_skip()
    N = 700
    case = "fp8 offset moves H=%d N=%d d=%d causal=%d" % (H, N, d, causal)
    note(case)
    rng = np.random.default_rng(9300 + d + causal)
    q = rng.standard_normal((1, H, N, d), dtype=np.float32) * 0.5
    k = rng.standard_normal((1, H, N, d), dtype=np.float32) * 0.1
    v = rng.standard_normal((1, H, N, d), dtype=np.float32)
    q[..., 0] = 4.0
    k[..., 0] = 0.0
    k[:, :, 200, 0] = 12.0
    k[:, :, 500, 0] = 30.0
    k[:, :, N - 3, 0] = 40.0
    k[:, :, 100, 0] = -30.0
    rt = lambda x: W.bf16_bits_to_f32(W.bf16_bits_rne(x))
    q, k, v = rt(q), rt(k), rt(v)
    O, L = _run_fp8(*_gpu_quant(q, k, v), 1.0, causal)
    _, deq = _oracle_quant(q, k, v)
    _check_rows(O, L, deq, 1.0, causal, np.arange(H * N), case)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(1, 8, 2, 300, 128, True), (2, 4, 1, 257, 64, False),
                                                 (1, 4, 1, 600, 64, True)])
def test_fp8_grouped_kv_heads(B, H, Hkv, N, d, causal):
    """fa_fwd_fp8_gqa: query head h reads K/V head h / (H/Hkv).  Against the
    oracle on the dequantized inputs with K/V repeated per query head, and bit
    for bit against fa_fwd_fp8 on the repeated quantized K/V."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    G = H // Hkv
    case = "fp8 gqa B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (B, H, Hkv, N, d, causal)
    note(case)
    q = _bf((B, H, N, d), 70 + N + d)
    k, v = _bf((B, Hkv, N, d), 71 + N + d), _bf((B, Hkv, N, d), 72 + N + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    q8, qs, k8, ks, v8t, vs = _gpu_quant_heads(q, k, v)
    O, L = _run_fp8(q8, qs, k8, ks, v8t, vs, scale, causal)
    # oracle side: dequantized K/V of the Hkv heads, repeated for each query head
    qc, qsc = mx.mx_quantize(q, axis=-1)
    kc, ksc = mx.mx_quantize(k, axis=-1)
    T = (N + 63) // 64
    vp = np.zeros((B * Hkv, T * 64, d), dtype=np.float32)
    vp[:, :N] = v.reshape(B * Hkv, N, d)
    vc, vsc = mx.mx_quantize(vp, axis=-2)
    vdq = mx.mx_dequantize(vc, vsc, axis=-2)[:, :N].reshape(B, Hkv, N, d)
    deq = (mx.mx_dequantize(qc, qsc), np.repeat(mx.mx_dequantize(kc, ksc), G, axis=1), np.repeat(vdq, G, axis=1))
    _check_rows(O, L, deq, scale, causal, np.arange(B * H * N), case)
    # the same bits as the multi-head kernel on repeated codes and scales
    rep = lambda t: t.reshape(B, Hkv, -1).repeat_interleave(G, dim=1).reshape(-1).contiguous()
    o2, l2 = fa.fwd_fp8(q8, qs, k8.repeat_interleave(G, dim=1).contiguous(),
                        ks.repeat_interleave(G, dim=1).contiguous(), rep(v8t), rep(vs),
                        scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert np.array_equal(o2.float().cpu().numpy(), O.astype(np.float32)) and \
        np.array_equal(l2.cpu().numpy(), L.astype(np.float32))


def _gpu_quant_heads(q, k, v):
    """GPU quantization of q [B,H,N,d] and k, v [B,Hkv,N,d]."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    q8, qs = fa.quantize_qk_fp8(upload(q, "bf16"))
    k8, ks = fa.quantize_qk_fp8(upload(k, "bf16"))
    v8t, vs = fa.quantize_v_fp8(upload(v, "bf16"))
    torch.cuda.synchronize()
    return q8, qs, k8, ks, v8t, vs


# ------------------------------------------------- incoherent processing
def _signs(d, seed):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1, 1).astype(np.int8)


def _gpu_quant_rot(x, signs):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    sd = torch.from_numpy(signs).cuda() if signs is not None else None
    x8, xs = fa.quantize_qk_fp8(upload(x, "bf16"), rotate=True, signs=sd)
    torch.cuda.synchronize()
    return x8, xs


@pytest.mark.parametrize("N,d,with_signs", [(100, 64, True), (300, 128, True), (65, 128, False), (1, 64, False)])
def test_rotated_quantizer_bit_exact(N, d, with_signs):
    """fa_quantize_qk_fp8_rotated: codes and scales of x diag(s) H_d equal the
    oracle's (rotation in float64, one rounding to float32, MX quantization)."""
    torch_or_skip()
    B, H = 2, 3
    note("fp8 rotated quantizer N=%d d=%d signs=%d" % (N, d, with_signs))
    s = _signs(d, N + d) if with_signs else None
    for x in (_bf((B, H, N, d), 11 + N, 2.0), _rotation_special_values((B, H, N, d), 12 + N)):
        g8, gs = (t.cpu().numpy() for t in _gpu_quant_rot(x, s))
        oc, osc = mx.mx_quantize(mx.rotate_rows(x, s), axis=-1)
        assert np.array_equal(g8, oc) and np.array_equal(gs, osc)


def _rotation_special_values(shape, seed):
    """bf16 rows for the rotated quantizer within its exactness condition
    (a row's magnitudes span fewer than 2^38): rows scaled by 2^k for k in
    [-40, 40), zero rows, rows of +-448, rows of float32/bf16 subnormals, rows
    with one channel x 2^10, and rows of equal values whose transform is zero
    except in one dim."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= (2.0 ** rng.integers(-40, 40, size=shape[:-1] + (1,))).astype(np.float32)
    flat = x.reshape(-1, shape[-1])
    flat[0::6] = 0.0
    flat[1::6] = np.float32(448.0) * np.sign(flat[1::6] + 0.5)
    flat[2::6] *= np.float32(1e-38)
    flat[3::6, 7] *= np.float32(1024.0)
    flat[4::6] = np.float32(3.0)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(flat.reshape(shape)))


def _outlier_inputs(B, H, N, d, seed, amp):
    """N(0,1) Q and K with the same two head dims (channels) multiplied by amp,
    the outlier-channel pattern incoherent processing targets; V N(0,1)."""
    q = np.random.default_rng(seed).standard_normal((B, H, N, d), dtype=np.float32)
    k = np.random.default_rng(seed + 1).standard_normal((B, H, N, d), dtype=np.float32)
    for ch in (5, d - 19):
        q[..., ch] *= np.float32(amp)
        k[..., ch] *= np.float32(amp)
    rt = lambda a: W.bf16_bits_to_f32(W.bf16_bits_rne(a))
    return rt(q), rt(k), _bf((B, H, N, d), seed + 2)


def _rotated_fp8(q, k, v, scale, causal, s):
    d = q.shape[-1]
    q8, qs = _gpu_quant_rot(q, s)
    k8, ks = _gpu_quant_rot(k, s)
    _, _, _, _, v8t, vs = _gpu_quant(q, k, v)
    return _run_fp8(q8, qs, k8, ks, v8t, vs, scale / d, causal)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 300, 128, True), (2, 2, 257, 64, False)])
def test_rotated_attention_within_derived_bound(B, H, N, d, causal):
    """Attention over rotated, quantized Q and K (scale / d) against the
    oracle's attention of the dequantized rotated inputs, at the bounds of
    the module docstring."""
    torch_or_skip()
    case = "fp8 rotated B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal)
    note(case)
    q, k, v = _outlier_inputs(B, H, N, d, 800 + N, 4.0)
    s = _signs(d, 5)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = _rotated_fp8(q, k, v, scale, causal, s)
    qc, qsc = mx.mx_quantize(mx.rotate_rows(q, s), axis=-1)
    kc, ksc = mx.mx_quantize(mx.rotate_rows(k, s), axis=-1)
    _, (_, _, vd) = _oracle_quant(q, k, v)
    deq = (mx.mx_dequantize(qc, qsc), mx.mx_dequantize(kc, ksc), vd)
    _check_rows(O, L, deq, scale / d, causal, np.arange(B * H * N), case)


@pytest.mark.parametrize("amp", [1.0, 6.0])
def test_rotation_lowers_outlier_channel_error(amp):
    """Against exact attention of the bf16 inputs: with two outlier channels
    (x6 in Q and K) the rotated path's error is well below block scaling
    alone; with none (x1) it is no worse than slightly above it."""
    torch_or_skip()
    B, H, N, d, causal = 1, 4, 512, 128, False
    q, k, v = _outlier_inputs(B, H, N, d, 900, amp)
    scale = float(np.float32(1 / math.sqrt(d)))
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    Ob, Lb = _run_fp8(*_gpu_quant(q, k, v), scale, causal)
    Or, Lr = _rotated_fp8(q, k, v, scale, causal, _signs(d, 7))
    rms = lambda a: float(np.sqrt(np.mean(a ** 2)))
    eb, er = rms(Ob - O_ref), rms(Or - O_ref)
    lb, lr = rms(Lb - L_ref), rms(Lr - L_ref)
    note("outlier amp %g: rms dO block-only %.3e rotated %.3e (x%.2f); rms dLSE %.3e vs %.3e"
         % (amp, eb, er, eb / er, lb, lr))
    if amp > 1:
        assert er < eb / 1.5 and lr < lb / 1.5
    else:
        assert er < 1.25 * eb and lr < 1.25 * lb
