"""The chunkwise-parallel form, re-derived in plain numpy fp64, equals the oracle.

The pages state only that within a chunk the updates become dense matrix
products and that only the passage from chunk to chunk is sequential (page
"Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV", section "Co stan
rekurencyjny zmienia przy serwowaniu", closing paragraph). The chunk algebra is
derived from the update of section "Gated DeltaNet: dodaj zanik" (per-key decay
as the Diag(a_t) reading). For a chunk of L tokens with start state S0 and
g_r = sum_{i<=r} log a_i:

    L_ri = beta_r sum_j k_r[j] k_i[j] exp(g_r[j] - g_i[j])      (i < r)
    T~   = (I + L)^-1 Diag(beta)
    W    = T~ (K * e^G),   U' = T~ V,   U = U' - W S0^T
    O    = (Q * e^G) S0^T + tril_incl((Q * e^G)(K * e^-G)^T) U
    S_L  = S0 Diag(e^{g_L}) + U^T (K * e^{g_L - G})

This test evaluates those formulas literally (explicit matrix inverse) and
checks them against the token-by-token oracle; with C = 1 they are one step of
the recurrence. It pins the chunk algebra that the GPU kernels implement.
"""
import numpy as np
import pytest

import oracle


def chunked_reference(q, k, v, alpha, beta, cu, S0, C, interval):
    T, H, dk = q.shape
    dv = v.shape[2]
    per_key = alpha.ndim == 3
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dv, dk))
    snaps = []
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        seq_snaps = []
        for h in range(H):
            S = S0[n, h].astype(np.float64).copy() if S0 is not None else np.zeros((dv, dk))
            hs = []
            for c0 in range(s, e, C):
                c1 = min(c0 + C, e)
                K = k[c0:c1, h].astype(np.float64)
                Q = q[c0:c1, h].astype(np.float64)
                V = v[c0:c1, h].astype(np.float64)
                b = beta[c0:c1, h].astype(np.float64)
                if per_key:
                    la = np.log(alpha[c0:c1, h].astype(np.float64))
                else:
                    la = np.repeat(np.log(alpha[c0:c1, h].astype(np.float64))[:, None], dk, axis=1)
                G = np.cumsum(la, axis=0)
                gL = G[-1]
                Kd, Ki, Qd, Kt = K * np.exp(G), K * np.exp(-G), Q * np.exp(G), K * np.exp(gL - G)
                Lm = np.tril(b[:, None] * (Kd @ Ki.T), -1)
                Tt = np.linalg.inv(np.eye(c1 - c0) + Lm) @ np.diag(b)
                W, Up = Tt @ Kd, Tt @ V
                U = Up - W @ S.T
                o[c0:c1, h] = Qd @ S.T + np.tril(Qd @ Ki.T) @ U
                S = S * np.exp(gL)[None, :] + U.T @ Kt
                if interval and (c1 - s) % interval == 0:
                    hs.append(S.copy())
            fin[n, h] = S
            seq_snaps.append(hs)
        for m in range(len(seq_snaps[0])):
            snaps.append(np.stack([seq_snaps[h][m] for h in range(H)]))
    snaps = np.stack(snaps) if snaps else np.zeros((0, H, dv, dk))
    return o, fin, snaps


def _inputs(rng, lens, H, dk, dv, per_key, with_state):
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    a_shape = (T, H, dk) if per_key else (T, H)
    alpha = (1 / (1 + np.exp(-(2.0 + rng.standard_normal(a_shape))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((len(lens), H, dv, dk))).astype(np.float32) if with_state else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, alpha, beta, cu, S0


def _rel(x, r):
    return np.abs(x - r).max() / max(np.abs(r).max(), 1e-30) if r.size else 0.0


@pytest.mark.parametrize("per_key", [0, 1])
@pytest.mark.parametrize("C", [1, 4, 8])
@pytest.mark.parametrize("d", [4, 8])
def test_chunked_form_equals_token_recurrence(per_key, C, d):
    rng = np.random.default_rng(100 + 10 * C + d + per_key)
    for T in (0, 1, 3, 7, 8, 9, 20):
        q, k, v, alpha, beta, cu, S0 = _inputs(rng, [T], 2, d, d + 1, per_key, True)
        o_r, f_r, s_r = oracle.run(q, k, v, alpha, beta, cu, S0, interval=8)
        o_c, f_c, s_c = chunked_reference(q, k, v, alpha, beta, cu, S0, C, 8)
        assert s_r.shape == s_c.shape
        assert _rel(o_c, o_r) < 1e-12 and _rel(f_c, f_r) < 1e-12 and _rel(s_c, s_r) < 1e-12


@pytest.mark.parametrize("per_key", [0, 1])
def test_chunked_form_varlen_with_empty_sequences(per_key):
    rng = np.random.default_rng(7 + per_key)
    lens = [0, 13, 8, 0, 25, 1]
    q, k, v, alpha, beta, cu, S0 = _inputs(rng, lens, 3, 8, 6, per_key, True)
    o_r, f_r, s_r = oracle.run(q, k, v, alpha, beta, cu, S0, interval=8)
    o_c, f_c, s_c = chunked_reference(q, k, v, alpha, beta, cu, S0, 4, 8)
    assert s_r.shape == s_c.shape == (sum(L // 8 for L in lens), 3, 6, 8)
    assert _rel(o_c, o_r) < 1e-12 and _rel(f_c, f_r) < 1e-12 and _rel(s_c, s_r) < 1e-12
    # an empty sequence leaves its state untouched
    assert np.array_equal(f_r[0], S0[0].astype(np.float64))
    assert np.array_equal(f_r[3], S0[3].astype(np.float64))


def test_chunk_of_one_is_one_token_step():
    """C = 1: L is empty, T~ = beta, and the chunk formulas are one update."""
    rng = np.random.default_rng(3)
    q, k, v, alpha, beta, cu, S0 = _inputs(rng, [1], 1, 5, 3, 1, True)
    o_c, f_c, _ = chunked_reference(q, k, v, alpha, beta, cu, S0, 1, 0)
    S = S0[0, 0].astype(np.float64) * alpha[0, 0].astype(np.float64)[None, :]
    kk = k[0, 0].astype(np.float64)
    u = beta[0, 0] * (v[0, 0].astype(np.float64) - S @ kk)
    S = S + np.outer(u, kk)
    np.testing.assert_allclose(f_c[0, 0], S, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o_c[0, 0], S @ q[0, 0].astype(np.float64), rtol=1e-13, atol=1e-15)
