"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Every check here runs on the CPU.  Each one is chosen so that a plausible
mistake in the oracle (a dropped scale, a wrong sign in the max subtraction,
log2 in place of ln, an off-by-one causal mask, a transposed operand, a
missing normalisation) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLD, "hand_example.json")) as f:
        return json.load(f)


def _hand_inputs(causal_rows=3, d=64, one_hot_values=False):
    """Three queries q_i = e0; keys k_j = s_j e0; values v_j = v_j e0.

    With scale = 1 every query sees the score row of the worked example.
    one_hot_values: v_j = e_j instead, so O row i returns the weights a_j.
    """
    g = _hand()
    s = np.array(g["scores"], dtype=np.float32)
    vals = np.array(g["values"], dtype=np.float32)
    q = np.zeros((1, 1, 3, d), np.float32)
    k = np.zeros((1, 1, 3, d), np.float32)
    v = np.zeros((1, 1, 3, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = s
    if one_hot_values:
        for j in range(3):
            v[0, 0, j, j] = 1.0
    else:
        v[0, 0, :, 0] = vals
    return q, k, v


@pytest.mark.parametrize("impl", ["c", "np"])
def test_hand_example_whole_row(impl):
    """notes section 8: O = 0.752 (0.7518 from the weights), l = 1.986."""
    g = _hand()
    pr, tol = g["printed"], g["printed_digits_tolerance"]
    q, k, v = _hand_inputs()
    f = oracle.attention_c if impl == "c" else oracle.attention_np
    O, L = f(q, k, v, 1.0, False)
    s0 = float(np.float32(g["scores"][0]))
    for i in range(3):
        assert abs(O[0, 0, i, 0] - pr["merged_O"]) < tol["three_decimals"]
        assert abs(O[0, 0, i, 0] - pr["whole_row_O"]) < tol["four_decimals"]
        assert np.all(O[0, 0, i, 1:] == 0.0)
        # LSE = m + ln l with m = 1.414, l = 1.986 (natural log)
        assert abs(math.exp(L[0, 0, i] - s0) - pr["merged_l"]) < tol["three_decimals"]
    # one-hot values return the softmax weights themselves
    q, k, v = _hand_inputs(one_hot_values=True)
    O, _ = f(q, k, v, 1.0, False)
    for j, a in enumerate(pr["whole_row_weights"]):
        assert abs(O[0, 0, 0, j] - a) < tol["four_decimals"]
    assert abs(O[0, 0, 0, :3].sum() - 1.0) < 1e-15


@pytest.mark.parametrize("impl", ["c", "np"])
def test_hand_example_causal_partials(impl):
    """With a causal mask row 1 sees only block 1 of section 8's split, so it
    returns the page's partial output O^(1) = 0.670 with l^(1) = 1.493;
    row 0 returns v_0; row 2 the merged 0.752."""
    g = _hand()
    pr, tol = g["printed"], g["printed_digits_tolerance"]
    q, k, v = _hand_inputs()
    f = oracle.attention_c if impl == "c" else oracle.attention_np
    O, L = f(q, k, v, 1.0, True)
    s0 = float(np.float32(g["scores"][0]))
    assert O[0, 0, 0, 0] == 1.0
    assert L[0, 0, 0] == s0
    assert abs(O[0, 0, 1, 0] - pr["block1_O"]) < tol["three_decimals"]
    assert abs(math.exp(L[0, 0, 1] - s0) - pr["block1_l"]) < tol["three_decimals"]
    assert abs(O[0, 0, 2, 0] - pr["merged_O"]) < tol["three_decimals"]


def test_hand_example_merge_forms():
    """Both merge forms, on both splits the page works by hand."""
    g = _hand()
    pr, tol = g["printed"], g["printed_digits_tolerance"]
    s = np.array(g["scores"])
    v = np.array(g["values"])[:, None]
    t3 = tol["three_decimals"]
    # section 8 split {1,2} | {3}
    trace = []
    O, l, m = oracle.online_merge_normalized(s, v, g["split_section8"], trace)
    assert abs(trace[0][1] - pr["block1_l"]) < t3
    assert abs(trace[0][2][0] - pr["block1_O"]) < t3
    assert abs(l - pr["merged_l"]) < t3 and abs(O[0] - pr["merged_O"]) < t3
    Od, ld, _ = oracle.online_merge_deferred(s, v, g["split_section8"])
    assert abs(ld - pr["merged_l"]) < t3 and abs(Od[0] - pr["merged_O"]) < t3
    # exercise 2 split {1} | {2,3}
    trace = []
    O, l, m = oracle.online_merge_normalized(s, v, g["split_exercise2"], trace)
    assert abs(trace[0][2][0] - pr["exercise2_block1_O"]) < t3
    assert abs(trace[0][1] - 1.0) < 1e-15
    assert abs(l - pr["exercise2_merged_l"]) < t3
    assert abs(O[0] - pr["exercise2_merged_O"]) < t3
    Od, ld, _ = oracle.online_merge_deferred(s, v, g["split_exercise2"])
    assert abs(Od[0] - pr["exercise2_merged_O"]) < t3


def test_numpy_demo_blocked_equals_whole():
    """aiqz.cc article, Python demo: block size 2 on the seed-0 4x3 problem
    agrees with whole-row attention to better than 1e-10 in float64."""
    with open(os.path.join(GOLD, "numpy_demo.json")) as f:
        g = json.load(f)
    rs = np.random.RandomState(g["seed"])
    N, d = g["N"], g["d"]
    Q, K, V = (rs.randn(N, d) for _ in range(3))
    O, _ = oracle.attention_np(Q[None, None], K[None, None], V[None, None], 1.0, False)
    splits = list(range(g["block"], N, g["block"]))
    for i in range(N):
        s = K @ Q[i]
        Ob, _, _ = oracle.online_merge_deferred(s, V, splits)
        assert np.abs(Ob - O[0, 0, i]).max() < g["max_abs_error_bound"]


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_constant_v(causal):
    B, H, N, d = 2, 3, 37, 8
    q, k = _rand((B, H, N, d), 1), _rand((B, H, N, d), 2)
    ones = np.ones((B, H, N, d), np.float32)
    O, _ = oracle.attention_c(q, k, ones, 0.35, causal)
    assert np.abs(O - 1.0).max() < 1e-14
    c = _rand((d,), 3)
    vc = np.broadcast_to(c, (B, H, N, d)).copy()
    O, _ = oracle.attention_c(q, k, vc, 0.35, causal)
    assert np.abs(O - c.astype(np.float64)).max() < 1e-14 * max(1.0, np.abs(c).max())


def test_causal_row0_and_single_key():
    B, H, N, d = 1, 2, 16, 8
    q, k, v = _rand((B, H, N, d), 4), _rand((B, H, N, d), 5), _rand((B, H, N, d), 6)
    scale = 0.25
    O, L = oracle.attention_c(q, k, v, scale, True)
    for h in range(H):
        assert np.array_equal(O[0, h, 0], v[0, h, 0].astype(np.float64))
        ref = scale * float(np.dot(q[0, h, 0].astype(np.float64), k[0, h, 0].astype(np.float64)))
        assert abs(L[0, h, 0] - ref) < 1e-14 * max(1.0, abs(ref))
    for causal in (False, True):
        O1, L1 = oracle.attention_c(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale, causal)
        assert np.array_equal(O1[:, :, 0], v[:, :, 0].astype(np.float64))


def test_key_permutation_invariance():
    B, H, N, d = 1, 2, 29, 8
    q, k, v = _rand((B, H, N, d), 7), _rand((B, H, N, d), 8), _rand((B, H, N, d), 9)
    perm = np.random.default_rng(10).permutation(N)
    O, L = oracle.attention_c(q, k, v, 0.3, False)
    Op, Lp = oracle.attention_c(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert np.abs(O - Op).max() < 1e-13
    assert np.abs(L - Lp).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_row_shift_of_keys(causal):
    """K' = K + 1 u^T: O is unchanged and LSE_i moves by scale <q_i, u>
    (softmax is unchanged by a per-row shift; notes section 5.1)."""
    B, H, N, d = 1, 1, 23, 4
    q = _rand((B, H, N, d), 11)
    k = _rand((B, H, N, d), 12)
    v = _rand((B, H, N, d), 13)
    u = np.array([0.5, -0.25, 1.0, 0.125], np.float32)   # exact in float32
    k2 = (k + u).astype(np.float32)
    scale = 0.5
    O, L = oracle.attention_c(q, k, v, scale, causal)
    O2, L2 = oracle.attention_c(q, k2, v, scale, causal)
    shift = scale * (q[0, 0].astype(np.float64) @ u.astype(np.float64))
    # k + u is rounded to float32, so compare to that rounding's size
    assert np.abs(O - O2).max() < 1e-5
    assert np.abs((L2 - L)[0, 0] - shift).max() < 1e-5


def test_linearity_in_v():
    B, H, N, d = 1, 2, 19, 8
    q, k = _rand((B, H, N, d), 14), _rand((B, H, N, d), 15)
    # values on a 1/64 grid, so 2*v1 - 3*v2 is exact in float32
    v1 = (np.round(_rand((B, H, N, d), 16) * 64) / 64).astype(np.float32)
    v2 = (np.round(_rand((B, H, N, d), 17) * 64) / 64).astype(np.float32)
    for causal in (False, True):
        O1, _ = oracle.attention_c(q, k, v1, 0.4, causal)
        O2, _ = oracle.attention_c(q, k, v2, 0.4, causal)
        O3, _ = oracle.attention_c(q, k, (2 * v1 - 3 * v2).astype(np.float32), 0.4, causal)
        assert np.abs(O3 - (2 * O1 - 3 * O2)).max() < 1e-12


def test_causal_row_is_prefix_attention():
    B, H, N, d = 1, 1, 12, 4
    q, k, v = _rand((B, H, N, d), 18), _rand((B, H, N, d), 19), _rand((B, H, N, d), 20)
    O, L = oracle.attention_c(q, k, v, 0.6, True)
    for i in range(N):
        Oi, Li = oracle.attention_np(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.6, False)
        assert np.abs(O[0, 0, i] - Oi[0, 0, i]).max() < 1e-13
        assert abs(L[0, 0, i] - Li[0, 0, i]) < 1e-13


def test_lse_bounds():
    B, H, N, d = 1, 2, 41, 8
    q, k, v = _rand((B, H, N, d), 21, 3.0), _rand((B, H, N, d), 22), _rand((B, H, N, d), 23)
    scale = 0.7
    for causal in (False, True):
        _, L = oracle.attention_c(q, k, v, scale, causal)
        s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        smax = s.max(-1)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        assert np.all(L >= smax - 1e-12)
        assert np.all(L <= smax + np.log(cnt) + 1e-12)


def test_extreme_scores_need_max_subtraction():
    """Scores 1000 and 0: exp(1000) overflows a double, so only a
    max-subtracted softmax returns v_0 and LSE = 1000 (cf-1.com write-up,
    section 3.1).  Scores -1000, -1000: exp underflows to 0 without the
    subtraction; the exact answer is the mean of v_0, v_1 with LSE = -1000+ln2."""
    d = 4
    q = np.zeros((1, 1, 2, d), np.float32)
    q[..., 0] = 1.0
    v = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0]], np.float32)[None, None]
    k = np.zeros((1, 1, 2, d), np.float32)
    k[0, 0, :, 0] = [1000.0, 0.0]
    for f in (oracle.attention_c, oracle.attention_np):
        O, L = f(q, k, v, 1.0, False)
        assert np.array_equal(O[0, 0, 0], v[0, 0, 0].astype(np.float64))
        assert L[0, 0, 0] == 1000.0
    k[0, 0, :, 0] = [-1000.0, -1000.0]
    for f in (oracle.attention_c, oracle.attention_np):
        O, L = f(q, k, v, 1.0, False)
        assert np.abs(O[0, 0, 0] - v[0, 0].mean(0)).max() < 1e-14
        assert abs(L[0, 0, 0] - (-1000.0 + math.log(2.0))) < 1e-12


def test_scale_closed_form():
    """Two keys with scores a, b (after scaling): O = sig(a-b) v0 + sig(b-a) v1,
    LSE = max(a,b) + ln(1 + exp(-|a-b|)).  scale = 0.5 halves the raw dots."""
    d = 2
    q = np.zeros((1, 1, 2, d), np.float32)
    q[..., 0] = 2.0
    k = np.zeros((1, 1, 2, d), np.float32)
    k[0, 0, :, 0] = [1.5, -0.75]            # raw dots 3.0 and -1.5
    v = np.array([[1.0, -1.0], [3.0, 10.0]], np.float32)[None, None]
    a, b = 0.5 * 3.0, 0.5 * -1.5
    w0 = 1.0 / (1.0 + math.exp(b - a))
    w1 = 1.0 / (1.0 + math.exp(a - b))
    for f in (oracle.attention_c, oracle.attention_np):
        O, L = f(q, k, v, 0.5, False)
        assert abs(O[0, 0, 0, 0] - (w0 * 1.0 + w1 * 3.0)) < 1e-14
        assert abs(O[0, 0, 0, 1] - (w0 * -1.0 + w1 * 10.0)) < 1e-14
        assert abs(L[0, 0, 0] - (a + math.log1p(math.exp(b - a)))) < 1e-14


def _brute_force(q, k, v, scale, causal):
    """Pure-Python loops over a tiny problem: weights exp(s_j)/sum exp(s),
    no max subtraction (scores stay small here)."""
    N, d = len(q), len(q[0])
    O, L = [], []
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        e = {j: math.exp(scale * sum(q[i][c] * k[j][c] for c in range(d))) for j in js}
        z = sum(e.values())
        O.append([sum(e[j] * v[j][c] for j in js) / z for c in range(d)])
        L.append(math.log(z))
    return O, L


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 2), (9, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(N, d, causal):
    q = _rand((1, 1, N, d), 30 + N)
    k = _rand((1, 1, N, d), 40 + N)
    v = _rand((1, 1, N, d), 50 + N)
    ref_O, ref_L = _brute_force(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.9, causal)
    for f in (oracle.attention_c, oracle.attention_np):
        O, L = f(q, k, v, 0.9, causal)
        assert np.abs(O[0, 0] - np.array(ref_O)).max() < 1e-13
        assert np.abs(L[0, 0] - np.array(ref_L)).max() < 1e-13


@pytest.mark.parametrize("N", [1, 2, 5, 9])
def test_block_merge_equals_whole_row_every_block_size(N):
    """Exercise 1 of the notes: the running merge keeps l and O exact after
    every block, for every block size and both merge forms."""
    d = 4
    rng = np.random.default_rng(60 + N)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = (rng.standard_normal((1, 1, N, d)) * 2).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    O, L = oracle.attention_c(q, k, v, 1.0, False)
    for i in range(N):
        s = k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64)
        for bs in range(1, N + 1):
            splits = list(range(bs, N, bs))
            Od, ld, md = oracle.online_merge_deferred(s, v[0, 0], splits)
            On, ln_, mn = oracle.online_merge_normalized(s, v[0, 0], splits)
            assert np.abs(Od - O[0, 0, i]).max() < 1e-12
            assert np.abs(On - O[0, 0, i]).max() < 1e-12
            assert abs(md + math.log(ld) - L[0, 0, i]) < 1e-12
            assert abs(mn + math.log(ln_) - L[0, 0, i]) < 1e-12
        # ragged split points too
        cuts = sorted(set(rng.integers(1, max(2, N), size=3).tolist()))
        Od, _, _ = oracle.online_merge_deferred(s, v[0, 0], [c for c in cuts if c < N])
        assert np.abs(Od - O[0, 0, i]).max() < 1e-12


def test_mistakes_are_caught():
    """The pins above fail on planted mistakes: a wrong-sign rescale and a
    block-local max in place of the running max (the classic bug the
    cf-1.com write-up, section 4.3, warns about)."""
    g = _hand()
    s = np.array(g["scores"])
    v = np.array(g["values"])[:, None]

    def merge_wrong_rescale(s, v, bounds, local_max):
        m, l, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        for a, b in oracle._blocks(len(s), bounds):
            mt = float(s[a:b].max())
            m_new = max(m, mt)
            r = np.exp((mt if local_max else m_new) - m) if np.isfinite(m) else 0.0
            p = np.exp(s[a:b] - m_new)
            l = r * l + p.sum()
            acc = r * acc + p @ v[a:b]
            m = m_new
        return acc / l

    good = oracle.online_merge_deferred(s[::-1].copy(), v[::-1].copy(), [1])[0][0]
    assert abs(good - g["printed"]["merged_O"]) < 5e-4
    for local in (False, True):
        bad = merge_wrong_rescale(s[::-1].copy(), v[::-1].copy(), [1], local)[0]
        assert abs(bad - g["printed"]["merged_O"]) > 5e-3


def test_c_and_numpy_oracles_agree_on_workloads():
    from io_aware_softmax_fwd_amd import workloads as W
    for cfg in (1, 2):
        x = W.make_inputs(cfg)
        w = x["workload"]
        Oc, Lc = oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal)
        On, Ln = oracle.attention_np(x["q"], x["k"], x["v"], w.scale, w.causal)
        assert np.abs(Oc - On).max() < 1e-12
        assert np.abs(Lc - Ln).max() < 1e-12


# --------------------------------------------------------------- Nq != Nk
def test_rectangular_rows_equal_last_rows_of_square_problem():
    """Query rows Q' = the last Nq rows of a square problem's Q: for both
    masks, every row of (Q', K, V) equals the matching last row of the square
    problem (causal aligns the last query with the last key)."""
    B, H, Nk, d = 1, 2, 37, 8
    q = _rand((B, H, Nk, d), 70)
    k = _rand((B, H, Nk, d), 71)
    v = _rand((B, H, Nk, d), 72)
    for Nq in (1, 5, 36, 37):
        for causal in (False, True):
            O_sq, L_sq = oracle.attention_c(q, k, v, 0.4, causal)
            for f in (oracle.attention_c, oracle.attention_np):
                O, L = f(q[:, :, Nk - Nq:].copy(), k, v, 0.4, causal)
                assert np.abs(O - O_sq[:, :, Nk - Nq:]).max() < 1e-13
                assert np.abs(L - L_sq[:, :, Nk - Nq:]).max() < 1e-13


def test_single_query_causal_sees_every_key():
    B, H, Nk, d = 2, 1, 50, 4
    q = _rand((B, H, 1, d), 73)
    k = _rand((B, H, Nk, d), 74)
    v = _rand((B, H, Nk, d), 75)
    Oc, Lc = oracle.attention_c(q, k, v, 0.7, True)
    On, Ln = oracle.attention_c(q, k, v, 0.7, False)
    assert np.array_equal(Oc, On) and np.array_equal(Lc, Ln)


@pytest.mark.parametrize("Nq,Nk", [(1, 7), (3, 8), (6, 6)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_rectangular(Nq, Nk, causal):
    d = 3
    q = _rand((1, 1, Nq, d), 80 + Nq)
    k = _rand((1, 1, Nk, d), 90 + Nk)
    v = _rand((1, 1, Nk, d), 95 + Nk)
    ql, kl, vl = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    for f in (oracle.attention_c, oracle.attention_np):
        O, L = f(q, k, v, 0.8, causal)
        for i in range(Nq):
            js = range(i + Nk - Nq + 1) if causal else range(Nk)
            e = {j: math.exp(0.8 * sum(ql[i][c] * kl[j][c] for c in range(d))) for j in js}
            z = sum(e.values())
            ref = [sum(e[j] * vl[j][c] for j in js) / z for c in range(d)]
            assert np.abs(O[0, 0, i] - np.array(ref)).max() < 1e-13
            assert abs(L[0, 0, i] - math.log(z)) < 1e-13


def test_causal_needs_enough_keys():
    q = _rand((1, 1, 4, 2), 1)
    k = _rand((1, 1, 3, 2), 2)
    for f in (oracle.attention_c, oracle.attention_np):
        with pytest.raises((ValueError, RuntimeError)):
            f(q, k, k, 1.0, True)


# ------------------------------------------------------ grouped K/V heads
@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3), (4, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_kv_heads(H, Hkv, causal):
    """The C oracle's head mapping (h -> h // (H // Hkv)) against the numpy
    oracle's explicit repetition of every K/V head, and each query head
    against a one-head problem over its K/V head."""
    B, Nq, Nk, d = 2, 9, 13, 4
    q = _rand((B, H, Nq, d), 100 + H)
    k = _rand((B, Hkv, Nk, d), 110 + Hkv)
    v = _rand((B, Hkv, Nk, d), 120 + Hkv)
    Oc, Lc = oracle.attention_c(q, k, v, 0.6, causal)
    On, Ln = oracle.attention_np(q, k, v, 0.6, causal)
    assert np.abs(Oc - On).max() < 1e-13 and np.abs(Lc - Ln).max() < 1e-13
    g = H // Hkv
    for b in range(B):
        for h in range(H):
            O1, L1 = oracle.attention_c(q[b:b + 1, h:h + 1], k[b:b + 1, h // g:h // g + 1],
                                        v[b:b + 1, h // g:h // g + 1], 0.6, causal)
            assert np.array_equal(O1[0, 0], Oc[b, h]) and np.array_equal(L1[0, 0], Lc[b, h])


def test_grouped_kv_heads_must_divide():
    q = _rand((1, 6, 4, 2), 1)
    k = _rand((1, 4, 4, 2), 2)
    with pytest.raises(ValueError):
        oracle.attention_c(q, k, k, 1.0, False)
