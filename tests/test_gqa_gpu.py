"""Parity of the grouped-K/V-head path (fa_fwd_gqa) with the fp64 oracle,
and its exact agreement with the multi-head path on repeated K/V heads."""
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


def _to_np(o, lse):
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _run_gqa(qd, kd, vd, scale, causal, splits, ws_pad=0):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, Nq, d = qd.shape
    ws = None
    if splits > 1:
        need = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, d, splits)
        full = torch.full((need + 2 * ws_pad,), 0xAB, dtype=torch.uint8, device="cuda")
        ws = full[ws_pad:ws_pad + need]
    o, lse = fa.fwd_gqa(qd, kd, vd, scale=scale, causal=causal, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None and ws_pad:
        h = full.cpu().numpy()
        assert np.all(h[:ws_pad] == 0xAB) and np.all(h[ws_pad + need:] == 0xAB)
    return o, lse


CASES = [
    # (B, H, Hkv, Nq, Nk, d, causal, splits)
    (2, 8, 2, 1, 3000, 128, True, 8),       # decoding, whole group in one tile
    (1, 32, 1, 1, 5000, 64, False, 16),     # multi-query decoding
    (1, 8, 2, 50, 700, 64, True, 1),        # packed tiles crossing head boundaries
    (1, 8, 2, 50, 700, 64, True, 4),
    (1, 6, 3, 37, 900, 128, True, 5),
    (1, 64, 4, 16, 2048, 128, True, 4),     # 16 heads of 16 rows: two packed tiles
    (2, 4, 2, 300, 300, 128, True, 1),      # long causal heads, tiles per head
    (2, 4, 2, 300, 300, 128, True, 3),
    (1, 8, 1, 513, 600, 64, True, 1),
    (1, 4, 2, 200, 333, 64, False, 1),      # non-causal, packed, ragged heads
    (1, 4, 2, 200, 333, 64, False, 4),
    (1, 2, 2, 130, 130, 128, True, 1),      # one query head per K/V head
    (1, 4, 1, 1, 1, 64, True, 1),
    (1, 4, 4, 3, 70, 128, True, 2),
    (1, 16, 2, 4, 1500, 128, True, 6),      # 8 heads x 4 positions: 32 rows, causal, one wave's rows
    (1, 8, 8, 1, 100, 128, True, 5),        # more chunks than key tiles, fewer tiles than waves
    (2, 32, 4, 1, 777, 64, False, 3),       # chunks of 4 or 5 tiles, ragged key tail
    (1, 64, 16, 2048, 2048, 64, True, 1),   # d = 64, 512 tiles of 256 rows: two blocks per wave
    (2, 64, 8, 1000, 1000, 64, False, 1),   # the same, packed 256-row tiles crossing heads
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,splits", CASES)
def test_gqa_matches_oracle(B, H, Hkv, Nq, Nk, d, causal, splits):
    case = "gqa B=%d H=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d splits=%d" % (
        B, H, Hkv, Nq, Nk, d, causal, splits)
    note(case)
    seed = 31 * H + 7 * Hkv + Nq + Nk + d + splits
    q = _bf((B, H, Nq, d), seed + 1)
    k = _bf((B, Hkv, Nk, d), seed + 2)
    v = _bf((B, Hkv, Nk, d), seed + 3)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = _run_gqa(upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), scale, causal,
                      splits, ws_pad=4096)
    O, L = _to_np(o, lse)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", case)


@pytest.mark.parametrize("H,Hkv,Nq,Nk,causal", [
    (8, 2, 50, 700, True), (8, 2, 300, 300, True), (8, 4, 200, 333, False), (16, 1, 1, 2000, True),
    (64, 8, 1000, 1000, False)])
def test_gqa_equals_multihead_on_repeated_heads(H, Hkv, Nq, Nk, causal):
    """One pass (no key split) gives every query row the same key tiles in
    the same order whichever rows share its workgroup, so fa_fwd_gqa must
    reproduce, bit for bit, fa_fwd_splitkv run on K/V with each head
    repeated H/Hkv times."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, d = 2, 64
    note("gqa == mha on repeated heads H=%d Hkv=%d Nq=%d Nk=%d causal=%d" % (H, Hkv, Nq, Nk, causal))
    q = upload(_bf((B, H, Nq, d), 5), "bf16")
    k = upload(_bf((B, Hkv, Nk, d), 6), "bf16")
    v = upload(_bf((B, Hkv, Nk, d), 7), "bf16")
    o1, l1 = _run_gqa(q, k, v, 0.125, causal, 1)
    kr = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    o2, l2 = fa.fwd_splitkv(q, kr, vr, scale=0.125, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_full_size_sampled_rows():
    """H=32 query heads over 8 K/V heads at N=16384, d=128, causal, with the
    amplified-row recipe (every K/V head read by four query heads); sampled
    rows against the oracle."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    w = W.WORKLOADS[4]
    Hkv = 8
    note("gqa full size: %s, Hkv=%d" % (w.describe(), Hkv))
    x = W.make_inputs(w)
    k = np.ascontiguousarray(x["k"][:, :Hkv])
    v = np.ascontiguousarray(x["v"][:, :Hkv])
    o, lse = _run_gqa(upload(x["q"], "bf16"), upload(k, "bf16"), upload(v, "bf16"), w.scale,
                      w.causal, 1)
    O, L = _to_np(o, lse)
    rows = W.sample_rows(w, 384, seed=41)
    O_ref, L_ref = oracle.attention_c(x["q"], k, v, w.scale, w.causal, rows=rows)
    assert_close(O.reshape(-1, w.d)[rows], L.reshape(-1)[rows], O_ref, L_ref, "bf16",
                 "gqa full size sampled rows")


def test_gqa_decode_default_splits():
    """The library's own split choice for a decoding step of 32 query heads
    over 8 K/V heads and 32768 keys."""
    torch = torch_or_skip()
    B, H, Hkv, Nq, Nk, d = 1, 32, 8, 1, 32768, 128
    note("gqa decode default splits")
    q = _bf((B, H, Nq, d), 21)
    k = _bf((B, Hkv, Nk, d), 22)
    v = _bf((B, Hkv, Nk, d), 23)
    scale = float(np.float32(1 / math.sqrt(d)))
    import io_aware_softmax_fwd_amd as fa
    o, lse = fa.fwd_gqa(upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), scale=scale,
                        causal=True, num_splits=None)
    torch.cuda.synchronize()
    O, L = _to_np(o, lse)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, True)
    assert_close(O, L, O_ref, L_ref, "bf16", "gqa decode default splits")
