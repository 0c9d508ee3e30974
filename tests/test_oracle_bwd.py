"""Pins of the backward oracle (oracle.kda_oracle.kda_recurrent_vjp).

The vector-Jacobian product is checked against two things that do not share
its code: central finite differences of the numpy forward recurrence
(kda_recurrent), and the closed form the recurrence takes at beta = 0, where
nothing is written and o_t = scale * q_t^T Diag(exp G_t) S_0.
"""
import numpy as np
import pytest

import oracle.kda_oracle as orc


def _inputs(B=1, T=24, H=2, K=5, V=4, seed=0, g_low=-5.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    g = g_low / (1.0 + np.exp(-rng.standard_normal((B, T, H, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    return q, k, v, g, beta


def _loss(q, k, v, g, beta, h0, do, df, scale, cu, l2):
    o, fin = orc.kda_recurrent(q, k, v, g, beta, scale, initial_state=h0, cu_seqlens=cu,
                               use_qk_l2norm=l2)
    return float(np.sum(o * do) + np.sum(fin * df))


@pytest.mark.parametrize("case", ["plain", "l2norm", "varlen"])
def test_vjp_matches_central_differences(case):
    """<grad, direction> equals the central difference of the loss along a
    random direction, for every input separately (step 1e-5, float64)."""
    B, T, H, K, V = 1, 24, 2, 5, 4
    q, k, v, g, beta = _inputs(B, T, H, K, V, seed=3)
    cu = np.array([0, 7, 7, 24]) if case == "varlen" else None
    nseq = 3 if case == "varlen" else B
    l2 = case == "l2norm"
    rng = np.random.default_rng(11)
    h0 = 0.3 * rng.standard_normal((nseq, H, K, V))
    do = rng.standard_normal((B, T, H, V))
    df = rng.standard_normal((nseq, H, K, V))
    scale = K ** -0.5
    grads = orc.kda_recurrent_vjp(q, k, v, g, beta, scale, do, df, h0, cu_seqlens=cu, use_qk_l2norm=l2)
    args = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "h0": h0}
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    eps = 1e-5
    for name, x in args.items():
        d = rng.standard_normal(x.shape)
        plus = dict(args)
        minus = dict(args)
        plus[name] = x + eps * d
        minus[name] = x - eps * d
        fd = (_loss(**plus, do=do, df=df, scale=scale, cu=cu, l2=l2)
              - _loss(**minus, do=do, df=df, scale=scale, cu=cu, l2=l2)) / (2 * eps)
        an = float(np.sum(grads[names[name]] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_vjp_beta_zero_closed_form():
    """beta = 0: o_t = s q_t^T D_t S0 and final = D_T S0 with D_t = Diag(exp G_t),
    G_t the inclusive cumulative gate. Then
      dq_t = s D_t S0 do_t,  dk = dv = 0,
      dg_m[d] = sum_{t >= m} s q_t[d] (D_t S0 do_t)[d] + (D_T S0 * dF)[d, :].sum(),
      dh0 = sum_t s D_t q_t do_t^T + D_T dF,
      dbeta_j = sum_{t >= j} s ((q_t * exp(G_t - G_j)) . k_j)(e_j . do_t)
                + sum_{d,v} dF[d, v] exp(G_T - G_j)[d] k_j[d] e_j[v],
    with e_j = v_j - (D_j S0)^T k_j (the write a token would make)."""
    B, T, H, K, V = 1, 10, 1, 4, 3
    q, k, v, g, _ = _inputs(B, T, H, K, V, seed=5)
    beta = np.zeros((B, T, H))
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((B, H, K, V))
    do = rng.standard_normal((B, T, H, V))
    dF = rng.standard_normal((B, H, K, V))
    s = 0.7
    r = orc.kda_recurrent_vjp(q, k, v, g, beta, s, do, dF, S0)
    G = np.cumsum(g[0, :, 0], axis=0)            # [T, K]
    S = S0[0, 0]
    F = dF[0, 0]
    D = np.exp(G)                                # [T, K]
    dq = np.stack([s * (D[t][:, None] * S) @ do[0, t, 0] for t in range(T)])
    assert np.allclose(r["dq"][0, :, 0], dq, atol=1e-12)
    assert np.abs(r["dk"]).max() < 1e-14 and np.abs(r["dv"]).max() < 1e-14
    per_t = np.stack([s * q[0, t, 0] * ((D[t][:, None] * S) @ do[0, t, 0]) for t in range(T)])
    fin_term = ((D[-1][:, None] * S) * F).sum(axis=1)
    dg = np.cumsum(per_t[::-1], axis=0)[::-1] + fin_term[None, :]
    assert np.allclose(r["dg"][0, :, 0], dg, atol=1e-12)
    dh0 = sum(s * np.outer(D[t] * q[0, t, 0], do[0, t, 0]) for t in range(T)) + D[-1][:, None] * F
    assert np.allclose(r["dh0"][0, 0], dh0, atol=1e-12)
    dbeta = np.zeros(T)
    for j in range(T):
        e = v[0, j, 0] - (D[j][:, None] * S).T @ k[0, j, 0]
        for t in range(j, T):
            dbeta[j] += s * np.dot(q[0, t, 0] * np.exp(G[t] - G[j]), k[0, j, 0]) * np.dot(e, do[0, t, 0])
        dbeta[j] += np.sum(F * (np.exp(G[-1] - G[j]) * k[0, j, 0])[:, None] * e[None, :])
    assert np.allclose(r["dbeta"][0, :, 0], dbeta, atol=1e-12)


def test_vjp_without_final_gradient_and_empty_segment():
    """d_final = None equals d_final = 0, and an empty segment gets dh0 = 0."""
    q, k, v, g, beta = _inputs(T=12, seed=8)
    rng = np.random.default_rng(4)
    cu = np.array([0, 5, 5, 12])
    h0 = rng.standard_normal((3, 2, 5, 4))
    do = rng.standard_normal(v.shape)
    a = orc.kda_recurrent_vjp(q, k, v, g, beta, 0.5, do, None, h0, cu_seqlens=cu)
    b = orc.kda_recurrent_vjp(q, k, v, g, beta, 0.5, do, np.zeros_like(h0), h0, cu_seqlens=cu)
    for n in a:
        assert np.array_equal(a[n], b[n])
    assert np.abs(a["dh0"][1]).max() == 0.0
