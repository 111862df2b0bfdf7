"""Long rows: one head of 131072 keys (2048 key tiles per row block).

The running max, the lazy offset and the fp32 row sums then see 128K keys;
inputs carry the amplified-row recipe (1 % of the Q and K rows scaled by 8,
seeded positions) so the offset moves far into the row.  Checked on sampled
rows (first and last rows, rows near tile edges and random ones) against the
oracle at the bf16 tolerances, through the single pass and the key split."""
import math

import numpy as np
import pytest

import oracle
from io_aware_softmax_fwd_amd import workloads as W

from gpu_util import assert_close, note, torch_or_skip, upload

pytestmark = pytest.mark.gpu

N = 131072


def _inputs(H, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, N, d), dtype=np.float32)
    k = rng.standard_normal((1, H, N, d), dtype=np.float32)
    v = rng.standard_normal((1, H, N, d), dtype=np.float32)
    for x in (q, k):
        rows = rng.choice(N, size=N // 100, replace=False)
        x[:, :, rows] *= 8.0
    rt = lambda x: W.bf16_bits_to_f32(W.bf16_bits_rne(x))
    return rt(q), rt(k), rt(v)


def _rows(H, seed):
    rng = np.random.default_rng(seed)
    picks = [0, 1, 63, 64, 127, 128, N - 129, N - 65, N - 2, N - 1]
    picks += list(rng.integers(0, N, 40))
    return np.unique(np.concatenate([h * N + np.array(picks) for h in range(H)]))


@pytest.mark.parametrize("d,causal", [(128, True), (64, True), (64, False)])
def test_long_rows(d, causal):
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    H = 2
    note("long rows: H=%d N=%d d=%d causal=%d" % (H, N, d, causal))
    q, k, v = _inputs(H, d, 8100 + d + causal)
    scale = float(np.float32(1 / math.sqrt(d)))
    rows = _rows(H, 8200 + d)
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, causal, rows=rows)
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    o, lse = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64).reshape(-1, d)[rows]
    L = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    assert_close(O, L, O_ref, L_ref, "bf16", "fa_fwd long rows d=%d causal=%d" % (d, causal))
    splits = 16
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(1, H, N, d, splits), dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64).reshape(-1, d)[rows]
    L = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    assert_close(O, L, O_ref, L_ref, "bf16", "fa_fwd_splitkv long rows d=%d causal=%d splits=%d" % (d, causal, splits))


@pytest.mark.parametrize("Hkv", [1, 8, 32])
def test_decode_full_size(Hkv):
    """The decoding step the benchmark times, at its size: one query row for
    each of 32 heads against 131072 keys (d=128, causal), K/V shared by
    32/Hkv query heads, with the chunk count the library suggests for this
    GPU (256 chunks for one K/V head).  Every row against the oracle."""
    torch = torch_or_skip()
    import io_aware_softmax_fwd_amd as fa
    B, H, d, nk = 1, 32, 128, N
    rng = np.random.default_rng(8300 + Hkv)
    rt = lambda x: W.bf16_bits_to_f32(W.bf16_bits_rne(x))
    q = rt(rng.standard_normal((B, H, 1, d), dtype=np.float32))
    k = rt(rng.standard_normal((B, Hkv, nk, d), dtype=np.float32))
    v = rt(rng.standard_normal((B, Hkv, nk, d), dtype=np.float32))
    scale = float(np.float32(1 / math.sqrt(d)))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = fa.fa_fwd_gqa_num_splits(B, H, Hkv, 1, nk, 1, cus)
    note("decode full size: H=%d Hkv=%d Nk=%d d=%d causal, %d chunks" % (H, Hkv, nk, d, splits))
    o, lse = fa.fwd_gqa(upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), scale=scale, causal=True,
                        num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_c(q, k, v, scale, True)
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    assert_close(O, L, O_ref, L_ref, "bf16", "fa_fwd_gqa decode Hkv=%d splits=%d" % (Hkv, splits))
