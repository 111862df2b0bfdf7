"""Parity of the key-split path (fa_fwd_splitkv) with the fp64 oracle."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, torch_or_skip, upload

pytestmark = pytest.mark.gpu


def _bf(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


def _run_split(q, k, v, scale, causal, splits, ws_pad=0):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    B, H, Nq, d = q.shape
    need = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, d, splits)
    ws = torch.full((need + 2 * ws_pad,), 0xAB, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, num_splits=splits,
                            workspace=ws[ws_pad:ws_pad + need])
    torch.cuda.synchronize()
    if ws_pad:
        wsh = ws.cpu().numpy()
        assert np.all(wsh[:ws_pad] == 0xAB) and np.all(wsh[ws_pad + need:] == 0xAB)
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    # (B, H, Nq, Nk, d, causal, splits)
    (2, 8, 1024, 1024, 64, False, 1),
    (2, 8, 1024, 1024, 64, False, 4),
    (2, 8, 1024, 1024, 64, False, 7),
    (1, 2, 513, 513, 128, True, 3),
    (1, 2, 513, 513, 128, True, 1),
    (1, 4, 1, 4096, 128, True, 16),
    (1, 4, 1, 4096, 128, False, 8),
    (1, 2, 100, 1000, 64, True, 5),
    (1, 2, 7, 5000, 64, False, 13),
    (1, 3, 130, 100, 128, False, 5),     # more chunks than key tiles
    (1, 1, 1, 1, 64, True, 2),
    (1, 2, 256, 300, 128, True, 6),
    # few rows: the merge splits a row's head dims over 8, 4 or 2 workgroups
    (1, 8, 1, 17000, 128, True, 256),
    (1, 8, 12, 3000, 128, True, 9),
    (1, 3, 50, 2000, 128, False, 11),
    (1, 16, 2, 2500, 64, True, 17),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,splits", CASES)
def test_splitkv_matches_oracle(B, H, Nq, Nk, d, causal, splits):
    case = "splitkv B=%d H=%d Nq=%d Nk=%d d=%d causal=%d splits=%d" % (B, H, Nq, Nk, d, causal, splits)
    note(case)
    seed = Nq * 7 + Nk + d + splits
    q = _bf((B, H, Nq, d), seed + 1)
    k = _bf((B, H, Nk, d), seed + 2)
    v = _bf((B, H, Nk, d), seed + 3)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = _run_split(q, k, v, scale, causal, splits, ws_pad=4096)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", case)


def test_splitkv_on_small_workload_matches_fa_fwd():
    """The split path on the B=2 H=8 N=1024 d=64 workload agrees with the
    single-pass kernel to the bf16 tolerance of the oracle (only the summation
    order differs)."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    w = W.WORKLOADS[2]
    x = W.make_inputs(w)
    qd, kd, vd = (upload(x[n], "bf16") for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
    o2, l2 = fa.fwd_splitkv(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal)
    for o, l, what in ((o1, l1, "fa_fwd"), (o2, l2, "fa_fwd_splitkv")):
        assert_close(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                     O_ref, L_ref, "bf16", "C2 " + what)


def test_splitkv_amplified_rows_decode():
    """Large score spreads (rows x8) with many chunks: the merge must keep
    exp(LSE_s - LSE) in range."""
    B, H, Nq, Nk, d = 1, 2, 3, 3000, 128
    q = _bf((B, H, Nq, d), 11, 8.0)
    k = _bf((B, H, Nk, d), 12)
    k[:, :, ::97] *= 8
    v = _bf((B, H, Nk, d), 13)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = _run_split(q, k, v, scale, True, 24)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, True)
    assert_close(O, L, O_ref, L_ref, "bf16", "amplified decode")
