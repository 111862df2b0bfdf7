"""Small grids: problems whose 128-row query tiles number at most 192 (three
quarters of the CUs) and whose rows see at least eight 64-key tiles run a
kernel whose four waves share 32 query rows and split the key tiles (wave w:
tiles w, w+4, ...), merging their partial results in LDS.  Every output row is
compared with the fp64 oracle at the bf16 tolerances: key-tile counts that
leave the waves uneven, ragged query and key tails, causal diagonals, both
head dims, grouped K/V heads with packed or per-head query tiles, and
Nq < Nk (decoding-like rows).  Shapes just above the threshold stay on the
128-row kernel and are checked the same way, so both sides of the switch are
covered."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, run, torch_or_skip, upload

pytestmark = pytest.mark.gpu


def _bf(shape, seed, amp=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(amp)
    return W.bf16_bits_to_f32(W.bf16_bits_rne(x))


# (B, H, N, d, causal): 8, 9, 10, 11 and many key tiles, ragged N
WS_SHAPES = [
    (1, 1, 512, 64, False), (1, 2, 513, 128, False), (1, 2, 600, 64, True), (1, 24, 1000, 64, True),
    (2, 3, 700, 128, True), (1, 1, 4100, 128, True), (2, 8, 1024, 64, True),
    (1, 4, 2047, 64, False), (3, 5, 1000, 128, False), (1, 7, 3001, 64, True),
]
# over the threshold (more than 192 workgroups of 128 rows): the 128-row kernel
REGULAR_SHAPES = [(1, 20, 1700, 128, True), (1, 40, 777, 64, False), (2, 16, 1025, 128, False),
                  (1, 25, 1000, 64, True)]


@pytest.mark.parametrize("B,H,N,d,causal", WS_SHAPES + REGULAR_SHAPES)
def test_square_against_oracle(B, H, N, d, causal):
    torch_or_skip()
    path = "ws" if (B * H * -(-N // 128) <= 192 and -(-N // 64) >= 8) else "128-row"
    case = "%s B=%d H=%d N=%d d=%d causal=%d" % (path, B, H, N, d, causal)
    note(case)
    seed = 31 * N + d + 7 * H + causal
    q, k, v = (_bf((B, H, N, d), seed + t, 2.0 if t < 2 else 1.0) for t in range(3))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run(q, k, v, scale, causal, "bf16")
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", case)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", [
    (1, 8, 2, 600, 600, 128, True),      # per-head causal tiles of 32 rows
    (1, 8, 2, 20, 900, 64, True),        # packed tiles crossing heads, Nq < Nk
    (2, 32, 4, 1, 5000, 128, True),      # a decoding step: one row per head
    (1, 6, 3, 77, 1300, 64, False),
])
def test_grouped_heads_against_oracle(B, H, Hkv, Nq, Nk, d, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    case = "ws gqa B=%d H=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d" % (B, H, Hkv, Nq, Nk, d, causal)
    note(case)
    seed = 17 * Nk + Nq + H
    q = _bf((B, H, Nq, d), seed + 1)
    k = _bf((B, Hkv, Nk, d), seed + 2)
    v = _bf((B, Hkv, Nk, d), seed + 3)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.fwd_gqa(upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), scale=scale,
                        causal=causal, num_splits=1)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal)
    assert_close(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 O_ref, L_ref, "bf16", case)


def test_small_grid_is_deterministic():
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, N, d = 2, 8, 1024, 64
    qd, kd, vd = (upload(_bf((B, H, N, d), 50 + t), "bf16") for t in range(3))
    outs = []
    for _ in range(3):
        o, lse = fa.fwd(qd, kd, vd, scale=0.125, causal=False)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy().view(np.int32)))
    for o, lse in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(lse, outs[0][1])
