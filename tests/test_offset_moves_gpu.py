"""The exponent offset of a row moving in the middle of the row.

The bf16 kernels take a tile's probabilities against the row's current
offset and move the offset (to the tile's row max, rescaling what was
accumulated) only when some lane's share of the tile's probability sum
exceeds 2^48 or is not finite.  These inputs force that move on chosen
tiles: keys whose score against every query sits far above all earlier
keys (by 69, 173 and 231 log2 units), one on a ragged last tile, and a key far
below the rest.  Results must still match the fp64 oracle at the bf16
tolerances, through the single-pass and the key-split entry points."""
import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, run, torch_or_skip, upload

pytestmark = pytest.mark.gpu


def _inputs(H, N, d, seed):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((1, H, N, d), dtype=np.float32) * 0.5)
    k = (rng.standard_normal((1, H, N, d), dtype=np.float32) * 0.1)
    v = rng.standard_normal((1, H, N, d), dtype=np.float32)
    q[..., 0] = 4.0                  # every query: the same large component
    k[..., 0] = 0.0
    k[:, :, 200, 0] = 12.0           # raw score 48 over earlier keys (tile 3)
    k[:, :, 500, 0] = 30.0           # raw score 120 (tile 7)
    k[:, :, N - 3, 0] = 40.0         # on the ragged last tile (raw score 160)
    k[:, :, 100, 0] = -30.0          # far below: weight underflows to 0
    rt = lambda x: W.bf16_bits_to_f32(W.bf16_bits_rne(x))
    return rt(q), rt(k), rt(v)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_single_pass(d, causal):
    torch_or_skip()
    H, N = 2, 700
    note("offset moves: single pass N=%d d=%d causal=%d" % (N, d, causal))
    q, k, v = _inputs(H, N, d, 9100 + d + causal)
    O, L = run(q, k, v, 1.0, causal, "bf16")
    O_ref, L_ref = oracle.attention_c(q, k, v, 1.0, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", "offset moves d=%d causal=%d" % (d, causal))
    # the largest visible key takes almost all the weight: O row ~ its V row
    # (key N-3 for every row when not causal; key 500 for causal rows before N-3)
    top = 500 if causal else N - 3
    rows = np.arange(510, N - 3) if causal else np.arange(0, N)
    np.testing.assert_allclose(O[0, 0, rows], np.broadcast_to(v[0, 0, top], O[0, 0, rows].shape),
                               atol=2e-2 * np.abs(v[0, 0, top]).max())


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_split(splits, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    H, N, d = 2, 700, 128
    note("offset moves: key split N=%d d=%d causal=%d splits=%d" % (N, d, causal, splits))
    q, k, v = _inputs(H, N, d, 9200 + splits + causal)
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(1, H, N, d, splits), dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd_splitkv(qd, kd, vd, scale=1.0, causal=causal, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = oracle.attention_c(q, k, v, 1.0, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", "offset moves split=%d causal=%d" % (splits, causal))


@pytest.mark.parametrize("H", [2, 40])      # 2: the small-grid kernel; 40: the 128-row kernel
@pytest.mark.parametrize("causal", [False, True])
def test_large_v_within_contract(H, causal):
    """fa_fwd promises finite, accurate O for max|v| < 2^48: with the offset
    lagging the row max the unnormalised accumulators reach about
    2^48 * keys * max|v| before a move.  V of magnitude 2^44 on the inputs
    that force offset moves (and whose earlier tiles carry probabilities far
    above 1 against a stale offset) must still match the oracle, whose error
    bound scales with max|O|."""
    torch_or_skip()
    N, d = 700, 128
    note("large V: H=%d N=%d d=%d causal=%d" % (H, N, d, causal))
    q, k, v = _inputs(H, N, d, 9400 + H + causal)
    v = W.bf16_bits_to_f32(W.bf16_bits_rne(v * np.float32(2.0 ** 44)))
    O, L = run(q, k, v, 1.0, causal, "bf16")
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    O_ref, L_ref = oracle.attention_c(q, k, v, 1.0, causal)
    assert_close(O, L, O_ref, L_ref, "bf16", "large V H=%d causal=%d" % (H, causal))
