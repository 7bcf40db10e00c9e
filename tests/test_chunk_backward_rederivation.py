"""The chunked backward algebra, re-derived in numpy fp64 with explicit
inverses, equals the oracle's token-by-token backward pass.

This is the specification the GPU backward kernels implement. For a chunk of
n tokens with start state S0, Gamma the in-chunk cumulative natural-log decay
(row r includes token r), a reference row c (any row: it cancels), and
  Kp = K e^(Gamma - Gamma_c), Km = K e^(Gamma_c - Gamma), Qp = Q e^(Gamma - Gamma_c)
  Ka = K e^Gamma, Qa = Q e^Gamma, Kt = K e^(Gamma_n - Gamma)
  P = Kp Km^T, L = strict_lower(Diag(beta) P), A = (I + L)^-1
  X = Diag(beta) Ka, Y = Diag(beta) V, W = A X, U' = A Y, U = U' - W S0^T
  Bm = lower(Qp Km^T), O = Qa S0^T + Bm U, S_n = S0 Diag(e^Gamma_n) + U^T Kt
the gradients given dO and dS_n are
  Z = Bm^T dO, dU = Z + Kt dS_n^T, dBm = lower(dO U^T)
  dQp = dBm Km, dQa = dO S0, dKm = dBm^T Qp + dL^T Diag(beta) Kp,
  dKt = U dS_n, dW = -dU S0, dA = dW X^T + dU Y^T, dX = A^T dW, dY = A^T dU,
  dL = strict_lower(-A^T dA A^T), dKp = Diag(beta) dL Km,
  dV = Diag(beta) dY, dbeta = rowsum(dY*V + dX*Ka + dL*P),
  dQ = dQp e^(Gamma-Gamma_c) + dQa e^Gamma,
  dK = dKp e^(Gamma-Gamma_c) + dKm e^(Gamma_c-Gamma) + Diag(beta) dX e^Gamma + dKt e^(Gamma_n-Gamma),
  dGamma = dQp*Qp + dQa*Qa + dKp*Kp - dKm*Km + (Diag(beta) dX)*Ka - dKt*Kt,
           plus colsum(dKt*Kt) + colsum(dS_n*S0)*e^Gamma_n on the last row,
  dlog a_i = sum_{r >= i} dGamma_r, da = dlog a / a (scalar gate: summed over channels)
and the gradient reaching the chunk's start state is
  dS0 = dS_n (Diag(e^Gamma_n) - Kt^T W) + E,  E = dO^T Qa - Z^T W,
a reverse affine scan over chunks with the transposed maps of the forward.
"""
import numpy as np
import pytest

import oracle


def _chunk_fwd(q, k, v, a, b, S0, ref):
    n = q.shape[0]
    G = np.cumsum(np.log(a), axis=0)                     # [n, dk]
    Gc = G[ref]
    Kp, Km, Qp = k * np.exp(G - Gc), k * np.exp(Gc - G), q * np.exp(G - Gc)
    Ka, Qa, Kt = k * np.exp(G), q * np.exp(G), k * np.exp(G[-1] - G)
    P = Kp @ Km.T
    L = np.tril(b[:, None] * P, -1)
    A = np.linalg.inv(np.eye(n) + L)
    X, Y = b[:, None] * Ka, b[:, None] * v
    W, Up = A @ X, A @ Y
    U = Up - W @ S0.T
    Bm = np.tril(Qp @ Km.T)
    O = Qa @ S0.T + Bm @ U
    Sn = S0 * np.exp(G[-1])[None, :] + U.T @ Kt
    return dict(G=G, Kp=Kp, Km=Km, Qp=Qp, Ka=Ka, Qa=Qa, Kt=Kt, P=P, A=A, X=X, Y=Y, W=W, U=U, Bm=Bm, O=O, Sn=Sn)


def _chunk_bwd(c, q, k, v, a, b, S0, dO, dSn, ref):
    Z = c["Bm"].T @ dO
    dU = Z + c["Kt"] @ dSn.T
    dBm = np.tril(dO @ c["U"].T)
    dQp, dQa = dBm @ c["Km"], dO @ S0
    dKt = c["U"] @ dSn
    dW = -dU @ S0
    dA = dW @ c["X"].T + dU @ c["Y"].T
    dX, dY = c["A"].T @ dW, c["A"].T @ dU
    dL = np.tril(-c["A"].T @ dA @ c["A"].T, -1)
    dKp = b[:, None] * (dL @ c["Km"])
    dKm = dBm.T @ c["Qp"] + dL.T @ (b[:, None] * c["Kp"])
    dV = b[:, None] * dY
    db = np.sum(dY * v, 1) + np.sum(dX * c["Ka"], 1) + np.sum(dL * c["P"], 1)
    G, Gc = c["G"], c["G"][ref]
    dKa = b[:, None] * dX
    dQ = dQp * np.exp(G - Gc) + dQa * np.exp(G)
    dK = dKp * np.exp(G - Gc) + dKm * np.exp(Gc - G) + dKa * np.exp(G) + dKt * np.exp(G[-1] - G)
    dG = dQp * c["Qp"] + dQa * c["Qa"] + dKp * c["Kp"] - dKm * c["Km"] + dKa * c["Ka"] - dKt * c["Kt"]
    dG[-1] += np.sum(dKt * c["Kt"], 0) + np.sum(dSn * S0, 0) * np.exp(G[-1])
    dloga = np.cumsum(dG[::-1], 0)[::-1]
    E = dO.T @ c["Qa"] - Z.T @ c["W"]
    return dQ, dK, dV, dloga / a, db, E


def chunked_backward(q, k, v, alpha, beta, cu, s0, d_o, d_f, C, per_key, ref_row):
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dalpha=np.zeros(alpha.shape), dbeta=np.zeros((T, H)), d_initial=np.zeros((N, H, dv, dk)))
    for n in range(N):
        for h in range(H):
            s, e = cu[n], cu[n + 1]
            S = s0[n, h].astype(np.float64)
            chunks = []
            for c0 in range(s, e, C):
                c1 = min(c0 + C, e)
                a = alpha[c0:c1, h].astype(np.float64)
                a = a if per_key else np.repeat(a[:, None], dk, 1)
                args = (q[c0:c1, h].astype(np.float64), k[c0:c1, h].astype(np.float64),
                        v[c0:c1, h].astype(np.float64), a, beta[c0:c1, h].astype(np.float64))
                ref = min(ref_row, c1 - c0 - 1)
                c = _chunk_fwd(*args, S, ref)
                chunks.append((c0, c1, args, S, c, ref))
                S = c["Sn"]
            dS = d_f[n, h].astype(np.float64)
            grads = []
            for c0, c1, args, S0, c, ref in reversed(chunks):
                dQ, dK, dV, da, db, E = _chunk_bwd(c, *args, S0, d_o[c0:c1, h].astype(np.float64), dS, ref)
                grads.append((c0, c1, dQ, dK, dV, da, db))
                dS = dS @ (np.diag(np.exp(c["G"][-1])) - c["Kt"].T @ c["W"]) + E
            out["d_initial"][n, h] = dS
            for c0, c1, dQ, dK, dV, da, db in grads:
                out["dq"][c0:c1, h], out["dk"][c0:c1, h], out["dv"][c0:c1, h] = dQ, dK, dV
                out["dalpha"][c0:c1, h] = da if per_key else da.sum(1)
                out["dbeta"][c0:c1, h] = db
    return out


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("C,ref_row", [(1, 0), (4, 1), (8, 3), (8, 7)])
def test_chunked_backward_equals_token_backward(per_key, C, ref_row):
    rng = np.random.default_rng(100 + C + ref_row)
    cu = [0, 13, 13, 14, 37]
    T, H, dk, dv, N = cu[-1], 2, 6, 4, len(cu) - 1
    f = np.float32
    q = (rng.standard_normal((T, H, dk)) * 0.5).astype(f)
    k = (rng.standard_normal((T, H, dk)) * 0.5).astype(f)
    v = rng.standard_normal((T, H, dv)).astype(f)
    alpha = rng.uniform(0.3, 1.0, (T, H, dk) if per_key else (T, H)).astype(f)
    beta = rng.uniform(0.0, 1.0, (T, H)).astype(f)
    s0 = (rng.standard_normal((N, H, dv, dk)) * 0.3).astype(f)
    d_o = rng.standard_normal((T, H, dv)).astype(f)
    d_f = rng.standard_normal((N, H, dv, dk)).astype(f)
    ref = oracle.backward(q, k, v, alpha, beta, cu, s0, d_o, d_f)
    got = chunked_backward(q, k, v, alpha, beta, cu, s0, d_o, d_f, C, per_key, ref_row)
    for name in ref:
        r = ref[name]
        err = np.max(np.abs(got[name] - r)) / max(np.max(np.abs(r)), 1e-300)
        assert err < 1e-10, (name, err)
