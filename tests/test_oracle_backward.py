"""Pins of the oracle's backward pass (kda_oracle_backward, fp64).

The hand-written reverse-mode steps are checked against things that do not
share them:
  - torch.autograd through a plain fp64 token loop written here from the
    update of the page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache
    KV" (trefon.com), section "Gated DeltaNet: dodaj zanik";
  - central finite differences of the forward oracle (already pinned on its
    own), on inputs that are exact multiples of the step;
  - the closed form at beta = 0, alpha = 1, where the state never changes;
  - linearity in the incoming gradients.
"""
import numpy as np
import pytest
import torch

import oracle



def _inputs(seed, cu, H, dk, dv, per_key, grid=None):
    rng = np.random.default_rng(seed)
    T = cu[-1]
    N = len(cu) - 1

    def r(*shape, lo=None, hi=None, scale=1.0):
        x = rng.uniform(lo, hi, shape) if lo is not None else rng.standard_normal(shape) * scale
        if grid:
            x = np.round(x / grid) * grid
        return x.astype(np.float32)

    q = r(T, H, dk, scale=0.5)
    k = r(T, H, dk, scale=0.5)
    v = r(T, H, dv)
    a = r(*((T, H, dk) if per_key else (T, H)), lo=0.55, hi=0.97)
    b = r(T, H, lo=0.05, hi=0.95)
    s0 = r(N, H, dv, dk, scale=0.3)
    d_o = r(T, H, dv)
    d_f = r(N, H, dv, dk, scale=0.5)
    return q, k, v, a, b, s0, d_o, d_f


def _autograd(q, k, v, a, b, cu, s0, d_o, d_f, per_key):
    """Plain fp64 token loop + torch.autograd."""
    t = {n: torch.tensor(x.astype(np.float64), dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, a=a, b=b, s0=s0).items()}
    loss = 0.0
    for n in range(len(cu) - 1):
        S = t["s0"][n]
        for tok in range(cu[n], cu[n + 1]):
            at = t["a"][tok][:, None, :] if per_key else t["a"][tok][:, None, None]
            S = S * at                                                     # S' = S Diag(a)
            p = torch.einsum("hij,hj->hi", S, t["k"][tok])
            u = t["b"][tok][:, None] * (t["v"][tok] - p)
            S = S + u[:, :, None] * t["k"][tok][:, None, :]
            o = torch.einsum("hij,hj->hi", S, t["q"][tok])
            loss = loss + (o * torch.tensor(d_o[tok].astype(np.float64), dtype=torch.float64)).sum()
        loss = loss + (S * torch.tensor(d_f[n].astype(np.float64), dtype=torch.float64)).sum()
    names = ["q", "k", "v", "a", "b", "s0"]
    grads = torch.autograd.grad(loss, [t[n] for n in names], allow_unused=True)
    return {n: (np.zeros(t[n].shape) if g is None else g.numpy()) for n, g in zip(names, grads)}


def _rel(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


CASES = [
    ([0, 7, 7, 8, 19], 2, 6, 4),     # empty and 1-token sequences, d_k != d_v
    ([0, 33], 1, 5, 5),              # several checkpoint segments (CK = 6)
]


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_equals_autograd(per_key, case):
    cu, H, dk, dv = CASES[case]
    q, k, v, a, b, s0, d_o, d_f = _inputs(10 + case, cu, H, dk, dv, per_key)
    g = oracle.backward(q, k, v, a, b, cu, s0, d_o, d_f)
    ref = _autograd(q, k, v, a, b, cu, s0, d_o, d_f, per_key)
    for mine, theirs in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dalpha", "a"), ("dbeta", "b"),
                         ("d_initial", "s0")):
        assert _rel(g[mine], ref[theirs]) < 1e-11, mine


def test_backward_bf16_inputs_equal_autograd():
    cu, H, dk, dv = [0, 5, 12], 2, 8, 8
    q, k, v, a, b, s0, d_o, d_f = _inputs(20, cu, H, dk, dv, True)
    to_bits = lambda x: (torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))  # noqa: E731
    from_bits = lambda u: (u.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    qb, kb, vb = to_bits(q), to_bits(k), to_bits(v)
    g = oracle.backward(qb, kb, vb, a, b, cu, s0, d_o, d_f)
    ref = _autograd(from_bits(qb), from_bits(kb), from_bits(vb), a, b, cu, s0, d_o, d_f, True)
    for mine, theirs in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dalpha", "a"), ("dbeta", "b"),
                         ("d_initial", "s0")):
        assert _rel(g[mine], ref[theirs]) < 1e-11, mine


@pytest.mark.parametrize("per_key", [False, True])
def test_backward_equals_finite_differences_of_forward_oracle(per_key):
    """Central differences of the forward oracle's fp64 outputs; every input is
    a multiple of h = 2^-10, so x +- h is exact in fp32."""
    h = 2.0 ** -10
    cu, H, dk, dv = [0, 6, 6, 15], 2, 4, 3
    q, k, v, a, b, s0, d_o, d_f = _inputs(30, cu, H, dk, dv, per_key, grid=h)

    def loss(q_, k_, v_, a_, b_, s0_):
        o, fin, _ = oracle.run(q_, k_, v_, a_, b_, cu, s0_, 0)
        return float(np.sum(o * d_o) + np.sum(fin * d_f))

    g = oracle.backward(q, k, v, a, b, cu, s0, d_o, d_f)
    base = dict(q_=q, k_=k, v_=v, a_=a, b_=b, s0_=s0)
    rng = np.random.default_rng(31)
    for name, gname in (("q_", "dq"), ("k_", "dk"), ("v_", "dv"), ("a_", "dalpha"), ("b_", "dbeta"),
                        ("s0_", "d_initial")):
        scale = max(np.max(np.abs(g[gname])), 1e-12)
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in base[name].shape)
            plus, minus = dict(base), dict(base)
            plus[name] = base[name].copy()
            minus[name] = base[name].copy()
            plus[name][idx] += np.float32(h)
            minus[name][idx] -= np.float32(h)
            fd = (loss(**plus) - loss(**minus)) / (2 * h)
            assert abs(fd - g[gname][idx]) <= 2e-4 * scale, (gname, idx, fd, g[gname][idx])


def test_backward_closed_form_identity_update():
    """beta = 0 and alpha = 1 leave S = S0 for every token, so o_t = S0 q_t:
    dq_t = S0^T do_t, dS0 = dSf + sum_t do_t q_t^T, dk = dv = 0, and with
    G_t = dSf + sum_{r >= t} do_r q_r^T: dbeta_t = (v_t - S0 k_t)^T G_t k_t,
    dalpha_t = sum_ij G_t[i,j] S0[i,j] (scalar gate)."""
    cu, H, dk, dv = [0, 10], 2, 5, 4
    q, k, v, _, _, s0, d_o, d_f = _inputs(40, cu, H, dk, dv, False)
    T = cu[-1]
    a = np.ones((T, H), np.float32)
    b = np.zeros((T, H), np.float32)
    g = oracle.backward(q, k, v, a, b, cu, s0, d_o, d_f)
    S0 = s0[0].astype(np.float64)
    for h in range(H):
        G = d_f[0, h].astype(np.float64).copy()
        for t in range(T - 1, -1, -1):
            G += np.outer(d_o[t, h].astype(np.float64), q[t, h].astype(np.float64))
            np.testing.assert_allclose(g["dq"][t, h], S0[h].T @ d_o[t, h], rtol=1e-12, atol=1e-12)
            u = v[t, h] - S0[h] @ k[t, h]
            np.testing.assert_allclose(g["dbeta"][t, h], u @ G @ k[t, h], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(g["dalpha"][t, h], np.sum(G * S0[h]), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(g["d_initial"][0, h], G, rtol=1e-12, atol=1e-12)
    assert np.all(g["dk"] == 0) and np.all(g["dv"] == 0)


def test_backward_linear_in_incoming_gradients():
    cu, H, dk, dv = [0, 9, 14], 2, 4, 4
    q, k, v, a, b, s0, d_o, d_f = _inputs(50, cu, H, dk, dv, True)
    g1 = oracle.backward(q, k, v, a, b, cu, s0, d_o, None)
    g2 = oracle.backward(q, k, v, a, b, cu, s0, np.zeros_like(d_o), d_f)
    g3 = oracle.backward(q, k, v, a, b, cu, s0, d_o, d_f)
    for n in g3:
        np.testing.assert_allclose(g1[n] + g2[n], g3[n], rtol=1e-12, atol=1e-12)


def test_backward_rejects_bad_inputs():
    cu, H, dk, dv = [0, 4], 1, 4, 4
    q, k, v, a, b, s0, d_o, d_f = _inputs(60, cu, H, dk, dv, False)
    with pytest.raises(ValueError):
        oracle.backward(q, k, v, a, b, cu, s0, d_o[:3], d_f)
    bad = a.copy()
    bad[0, 0] = 1.5
    with pytest.raises(ValueError):
        oracle.backward(q, k, v, bad, b, cu, s0, d_o, d_f)
