"""Pins of the backward oracle (oracle.attention_bwd_c / attention_bwd_np).

The pages give no gradient formulas (only the recomputation strategy), so
the gradients are pinned to the forward oracle, which is pinned to the pages
itself: central finite differences of L = sum(dO * O) in every direction
tested, plus the identities the softmax fixes (key gradients sum to zero,
value gradients sum to the summed upstream gradient, identical keys give no
query gradient) and closed forms for uniform attention.  Planted mistakes
(a dropped softmax-Jacobian term, a missing scale, a transposed product, a
missing causal mask) each fail the finite-difference pin.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, dO, scale, causal):
    O, _ = oracle.attention_np(q, k, v, scale, causal)
    return float((O * dO).sum())


def _fd_check(bwd, q, k, v, dO, scale, causal, seed=0, eps=1e-5):
    """Largest relative mismatch between <grad, E> and the central
    difference of L along a random direction E, over Q, K and V."""
    grads = bwd(q, k, v, dO, scale, causal)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for which in range(3):
        E = rng.standard_normal(q.shape)
        args = [q, k, v]
        plus = list(args)
        minus = list(args)
        plus[which] = args[which] + eps * E
        minus[which] = args[which] - eps * E
        fd = (_loss(*plus, dO, scale, causal) - _loss(*minus, dO, scale, causal)) / (2 * eps)
        an = float((grads[which] * E).sum())
        worst = max(worst, abs(fd - an) / max(1e-12, abs(fd), abs(an)))
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d,scale", [(1, 2, 7, 5, 0.7), (2, 1, 12, 8, 0.35), (1, 1, 1, 4, 1.0),
                                           (1, 1, 33, 3, 1.3)])
def test_bwd_matches_finite_differences(causal, B, H, N, d, scale):
    q, k, v, dO = (_rand((B, H, N, d), s) for s in (1, 2, 3, 4))
    for seed in range(3):
        assert _fd_check(oracle.attention_bwd_np, q, k, v, dO, scale, causal, seed) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_every_element_by_finite_differences(causal):
    """Element-by-element central differences on a tiny problem, so that no
    single entry can be wrong while the random directions still agree."""
    B, H, N, d, scale = 1, 1, 4, 3, 0.9
    q, k, v, dO = (_rand((B, H, N, d), s) for s in (11, 12, 13, 14))
    grads = oracle.attention_bwd_np(q, k, v, dO, scale, causal)
    eps = 1e-6
    for which in range(3):
        for idx in np.ndindex(q.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (_loss(*args_p, dO, scale, causal) - _loss(*args_m, dO, scale, causal)) / (2 * eps)
            assert abs(fd - grads[which][idx]) < 1e-8, (which, idx)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 64), (2, 3, 37, 16), (1, 2, 130, 64)])
def test_bwd_c_matches_numpy(causal, B, H, N, d):
    x = [_rand((B, H, N, d), s).astype(np.float32) for s in (21, 22, 23, 24)]
    c = oracle.attention_bwd_c(*x, 0.125, causal)
    n = oracle.attention_bwd_np(*x, 0.125, causal)
    for a, b in zip(c, n):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_bwd_c_head_subset():
    B, H, N, d = 2, 3, 20, 8
    x = [_rand((B, H, N, d), s).astype(np.float32) for s in (31, 32, 33, 34)]
    full = oracle.attention_bwd_c(*x, 0.3, True)
    heads = np.array([4, 0, 5])
    part = oracle.attention_bwd_c(*x, 0.3, True, heads=heads)
    for f, p in zip(full, part):
        fr = f.reshape(B * H, N, d)
        for t, h in enumerate(heads):
            assert np.array_equal(fr[h], p[t])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_softmax_identities(causal):
    """Rows of P sum to one and rows of dS sum to zero, so for every head
    sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    B, H, N, d = 2, 2, 25, 6
    x = [_rand((B, H, N, d), s).astype(np.float32) for s in (41, 42, 43, 44)]
    dQ, dK, dV = oracle.attention_bwd_c(*x, 0.5, causal)
    dO = x[3].astype(np.float64)
    assert np.abs(dV.sum(axis=2) - dO.sum(axis=2)).max() < 1e-12
    assert np.abs(dK.sum(axis=2)).max() < 1e-12


def test_bwd_single_key_and_identical_keys():
    """N = 1: O = v_0 whatever q and k are, so dQ = dK = 0 and dV = dO.
    Identical keys: every row's softmax is uniform whatever q is, so dQ = 0."""
    x = [_rand((1, 2, 1, 8), s).astype(np.float32) for s in (51, 52, 53, 54)]
    dQ, dK, dV = oracle.attention_bwd_c(*x, 0.9, False)
    assert np.abs(dQ).max() == 0 and np.abs(dK).max() == 0
    assert np.array_equal(dV, x[3].astype(np.float64))
    q = _rand((1, 1, 9, 4), 55).astype(np.float32)
    k = np.repeat(_rand((1, 1, 1, 4), 56).astype(np.float32), 9, axis=2)
    v, dO = (_rand((1, 1, 9, 4), s).astype(np.float32) for s in (57, 58))
    dQ, _, _ = oracle.attention_bwd_c(q, k, v, dO, 0.7, False)
    assert np.abs(dQ).max() < 1e-14
    # causal row 0 sees one key only
    dQc, _, _ = oracle.attention_bwd_c(q, _rand((1, 1, 9, 4), 59).astype(np.float32), v, dO, 0.7, True)
    assert np.abs(dQc[0, 0, 0]).max() == 0


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_uniform_attention_closed_form(causal):
    """q = 0 makes every visible score 0: P_ij = 1/|J_i|, so
    dV_j = sum_{i sees j} dO_i / |J_i| (|J_i| = N, or i + 1 when causal)."""
    N, d = 11, 5
    q = np.zeros((1, 1, N, d), dtype=np.float32)
    k, v, dO = (_rand((1, 1, N, d), s).astype(np.float32) for s in (61, 62, 63))
    _, _, dV = oracle.attention_bwd_c(q, k, v, dO, 1.0, causal)
    g = dO[0, 0].astype(np.float64)
    for j in range(N):
        rows = range(j, N) if causal else range(N)
        want = sum(g[i] / ((i + 1) if causal else N) for i in rows)
        assert np.abs(dV[0, 0, j] - want).max() < 1e-13


def _planted(kind):
    """attention_bwd_np with one deliberate mistake."""
    def bwd(q, k, v, dO, scale, causal):
        B, H, N, d = q.shape
        dQ, dK, dV = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, h] @ k[b, h].T)
                if causal and kind != "no_mask":
                    s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = dO[b, h] @ v[b, h].T
                if kind == "no_jacobian_term":
                    ds = p * dp
                else:
                    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dV[b, h] = (p @ dO[b, h]) if kind == "dv_untransposed" else (p.T @ dO[b, h])
                dQ[b, h] = scale * ((ds.T if kind == "dq_transposed" else ds) @ k[b, h])
                dK[b, h] = (1.0 if kind == "dk_no_scale" else scale) * (ds.T @ q[b, h])
        return dQ, dK, dV
    return bwd


@pytest.mark.parametrize("kind", ["no_jacobian_term", "dv_untransposed", "dq_transposed",
                                  "dk_no_scale", "no_mask"])
def test_planted_backward_mistakes_are_caught(kind):
    causal = kind == "no_mask"
    q, k, v, dO = (_rand((1, 2, 7, 5), s) for s in (71, 72, 73, 74))
    assert _fd_check(_planted(kind), q, k, v, dO, 0.7, causal) > 1e-3
