"""Every row of the three large workloads against the fp64 oracle.

C3 (B=4, H=16, N=4096, d=128, causal), C4 (B=1, H=32, N=16384, d=128,
causal, 1 % of the Q and K rows x8) and C5 (B=1, H=16, N=32749, d=64, a
ragged last tile) are run through fa_fwd in the launch configuration the
benchmark times, and all B*H*N output rows and log-sum-exps are compared
element by element with the plain three-step attention in IEEE double.  The
method is exact up to rounding (notes page, section 7.2, Theorem 1), so the
whole output must match at the bf16 tolerances: max|dO| <= 2e-2 max|O| and
max|dLSE| <= 1e-2.  The oracle takes about 3, 27 and 54 s on 16 host
threads; this file is collected after the faster GPU tests.
"""
import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, run, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_workload_every_row(cfg):
    torch_or_skip()
    w = W.WORKLOADS[cfg]
    note("workload C%d, every row: %s" % (cfg, w.describe()))
    x = W.make_inputs(w)
    O, L = run(x["q"], x["k"], x["v"], w.scale, w.causal, w.dtype)
    O_ref, L_ref = oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal)
    assert O.shape == O_ref.shape and L.shape == L_ref.shape
    assert_close(O, L, O_ref, L_ref, w.dtype, "C%d all %d rows" % (cfg, w.B * w.H * w.N))
    if w.amplify:
        # the rows whose query was amplified (largest scores, most offset moves)
        amp = np.zeros((w.B, w.H, w.N), bool)
        rows = W._amplified_rows(1000 * cfg + 4, w.B, w.H, w.N)
        for b in range(w.B):
            for h in range(w.H):
                amp[b, h, rows[b][h]] = True
        assert int(amp.sum()) == w.B * w.H * round(0.01 * w.N)
        note("C%d amplified query rows: %d, max|dO| there %.3e, max|dLSE| there %.3e" % (
            cfg, int(amp.sum()), float(np.abs(O - O_ref)[amp].max()), float(np.abs(L - L_ref)[amp].max())))


# ------------------------------------------------------------- backward
def test_bwd_every_head_c3():
    """fa_fwd then fa_bwd on C3 (B=4, H=16, N=4096, d=128, causal; dO drawn
    N(0,1) with seed 3006): dQ, dK and dV of all 64 heads against the
    oracle's gradients, within 2e-2 of each gradient's largest magnitude
    (about 30 s of oracle on 16 host threads)."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    from gpu_util import upload
    w = W.WORKLOADS[3]
    note("bwd C3 every head: %s" % w.describe())
    x = W.make_inputs(w)
    g = np.random.default_rng(1000 * 3 + 6).standard_normal(x["q"].shape, dtype=np.float32)
    g = W.bf16_bits_to_f32(W.bf16_bits_rne(g))
    qd, kd, vd, gd = (upload(a, "bf16") for a in (x["q"], x["k"], x["v"], g))
    o, lse = fa.fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, gd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    ref = oracle.attention_bwd_c(x["q"], x["k"], x["v"], g, w.scale, w.causal)
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        err, mx = float(np.abs(a - b).max()), float(np.abs(b).max())
        note("C3 bwd every head %s: max|err|=%.3e max|ref|=%.3e ratio=%.2e" % (name, err, mx, err / mx))
        assert np.all(np.isfinite(a)) and err <= 2e-2 * mx


# ------------------------------------------------------------------ fp8
def _fp8_bounds_head(qd, kd, vd, scale, causal, O_ref):
    """The per-element O bound and per-row LSE bound of tests/test_fp8_gpu.py
    for every row of one head, as whole-head float64 matrices: with weights
    w_ij and per-key rounding allowance e_ij = max(2^-4 w_ij, 2^-10 / l_i),
    sigma_ic^2 = sum_j e_ij^2 / 3 * (v_jc - O_ic)^2, expanded into products."""
    s = scale * (qd.astype(np.float64) @ kd.astype(np.float64).T)
    if causal:
        s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    wts = p / l
    e2 = np.maximum(2.0 ** -4 * wts, 2.0 ** -10 / l) ** 2 / 3
    if causal:
        e2 = np.where(np.tril(np.ones(s.shape, dtype=bool)), e2, 0.0)
    vv = vd.astype(np.float64)
    var = e2 @ (vv * vv) - 2 * O_ref * (e2 @ vv) + O_ref * O_ref * e2.sum(axis=1, keepdims=True)
    vmax = np.abs(vv).max(axis=0)[None, :]
    if causal:   # the largest |v| among each row's visible keys
        vmax = np.maximum.accumulate(np.abs(vv), axis=0)
    ob = 8 * np.sqrt(np.maximum(var, 0.0)) + 2.0 ** -8 * np.abs(O_ref) + 3e-4 * vmax
    lb = 8 * np.sqrt(e2.sum(axis=1)) + 1e-3
    return ob, lb


@pytest.mark.parametrize("cfg", [2, 3])
def test_fp8_every_row(cfg):
    """fa_fwd_fp8 on the MX-quantized inputs of C2 and C3, every row against
    the oracle's attention of the dequantized inputs, at the fp8 bounds
    (hard pin, statistical model and accumulation assumption of
    tests/test_fp8_gpu.py)."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    from oracle import mx_fp8 as mx
    from gpu_util import upload
    w = W.WORKLOADS[cfg]
    note("fp8 C%d every row: %s" % (cfg, w.describe()))
    x = W.make_inputs(w)
    qd8, qs = fa.quantize_qk_fp8(upload(x["q"], "bf16"))
    kd8, ks = fa.quantize_qk_fp8(upload(x["k"], "bf16"))
    v8t, vs = fa.quantize_v_fp8(upload(x["v"], "bf16"))
    o, lse = fa.fwd_fp8(qd8, qs, kd8, ks, v8t, vs, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    B, H, N, d = w.B, w.H, w.N, w.d
    qdq = mx.mx_dequantize(*mx.mx_quantize(x["q"], axis=-1))
    kdq = mx.mx_dequantize(*mx.mx_quantize(x["k"], axis=-1))
    T = (N + 63) // 64
    vp = np.zeros((B * H, T * 64, d), dtype=np.float32)
    vp[:, :N] = x["v"].reshape(B * H, N, d)
    vdq = mx.mx_dequantize(*mx.mx_quantize(vp, axis=-2), axis=-2)[:, :N].reshape(B, H, N, d)
    O_ref, L_ref = oracle.attention_c(qdq, kdq, vdq, w.scale, w.causal)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            ob, lb = _fp8_bounds_head(qdq[b, h], kdq[b, h], vdq[b, h], w.scale, w.causal, O_ref[b, h])
            eo = np.abs(O[b, h] - O_ref[b, h])
            el = np.abs(L[b, h] - L_ref[b, h])
            worst_o = max(worst_o, float((eo / ob).max()))
            worst_l = max(worst_l, float((el / lb).max()))
    note("fp8 C%d every row: worst dO/bound %.3f, worst dLSE/bound %.3f" % (cfg, worst_o, worst_l))
    assert worst_o <= 1.0 and worst_l <= 1.0
