"""Pins of the fp64 CPU oracle against facts the pages and the mathematics fix.

Every test here runs on the CPU. Each targets a plausible mistake in the oracle
(dropped decay, wrong sign of the delta term, read-out before the update, a
transposed state, snapshot off-by-one, cu_seqlens indexing):

  * identity (alpha=1, beta=0 leaves S unchanged) and the fixed point (a state
    that already maps k to v is not changed) -- page "Modele hybrydowe: co Gated
    DeltaNet zastępuje w cache KV", section "Reguła delta: zapisz poprawkę, nie
    sumę";
  * exact recall with orthonormal keys (the delta rule overwrites the stored
    association) -- same section;
  * reduction to causal linear attention with decay when keys are mutually
    orthogonal and S0 = 0 -- section "Atencja liniowa: stan o stałym rozmiarze";
  * channel-uniform per-key gate == scalar gate -- section "Gated DeltaNet: dodaj
    zanik";
  * pure decay sigma(5)^t, against the page-1 figures (alpha-gate bias +5 gives
    ~0.993; the product of alpha over 950 tokens is of order 1e-3) -- page
    "kda-graft" (ailist.pro), sections "Идея и архитектура" and "Атрибуция";
  * snapshot placement and packing with exact integer arithmetic, and prefix
    reuse from a snapshot -- section "Co stan rekurencyjny zmienia przy
    serwowaniu", item 1;
  * the literal matrix product form of the update evaluated in exact rational
    arithmetic on a tiny case.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x):
    """float32 values that are exactly representable in bf16 -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def rand_inputs(rng, T, H, dk, dv, per_key, n_seqs=1):
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    a_shape = (T, H, dk) if per_key else (T, H)
    alpha = (1.0 / (1.0 + np.exp(-(3.0 + rng.standard_normal(a_shape))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((n_seqs, H, dv, dk))).astype(np.float32)
    return q, k, v, alpha, beta, s0


@pytest.mark.parametrize("per_key", [0, 1])
def test_identity_alpha_one_beta_zero(per_key):
    rng = np.random.default_rng(1)
    T, H, dk, dv = 37, 2, 8, 5
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, per_key)
    alpha[:] = 1.0
    beta[:] = 0.0
    o, fin, _ = oracle.run(q, k, v, alpha, beta, [0, T], s0)
    assert np.array_equal(fin, s0.astype(np.float64))
    expect = np.einsum("hij,thj->thi", s0[0].astype(np.float64), q.astype(np.float64))
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_exact_recall_orthonormal_keys(dtype):
    """alpha=1, beta=1, n <= d_k orthonormal keys written in turn over ANY start
    state: the final state maps every k_i to its v_i."""
    rng = np.random.default_rng(2)
    dk, dv, H = 64, 24, 1
    # Sylvester Hadamard rows / 8 are orthonormal and exact in bf16 (+-1/8).
    Hm = np.array([[1.0]])
    while Hm.shape[0] < dk:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    rows = rng.permutation(dk)[:40]
    K = (Hm[rows] / 8.0).astype(np.float32)
    T = K.shape[0]
    k = K[:, None, :].copy()
    V = np.round(rng.standard_normal((T, dv)) * 8) / 8  # exact in bf16
    v = V.astype(np.float32)[:, None, :]
    q = k.copy()
    s0 = (rng.standard_normal((1, H, dv, dk))).astype(np.float32)  # not symmetric, dv != dk
    alpha = np.ones((T, H), np.float32)
    beta = np.ones((T, H), np.float32)
    if dtype == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    _, fin, _ = oracle.run(q, k, v, alpha, beta, [0, T], s0)
    S = fin[0, 0]
    recalled = S @ K.astype(np.float64).T           # [dv, T]: S k_i
    np.testing.assert_allclose(recalled, V.T, rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_key", [0, 1])
def test_reduces_to_decayed_linear_attention(per_key):
    """S0 = 0, beta = 1 and keys on distinct one-hot channels: the delta term
    S' k_t is always zero, so u_t = v_t and
        o_t = sum_{i<=t} v_i ((k_i * gamma_t / gamma_i) . q_t),
    gamma_t = prod_{j<=t} a_j (elementwise). With alpha = 1 this is plain causal
    linear attention."""
    rng = np.random.default_rng(3)
    T, H, dk, dv = 14, 1, 16, 6
    chans = rng.permutation(dk)[:T]
    k = np.zeros((T, H, dk), np.float32)
    k[np.arange(T), 0, chans] = rng.choice([-1.0, 1.0], size=T)
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    beta = np.ones((T, H), np.float32)
    for alpha_one in (True, False):
        if alpha_one:
            alpha = np.ones((T, H, dk) if per_key else (T, H), np.float32)
        else:
            shape = (T, H, dk) if per_key else (T, H)
            alpha = rng.uniform(0.5, 1.0, size=shape).astype(np.float32)
        o, fin, _ = oracle.run(q, k, v, alpha, beta, [0, T])
        a = alpha.astype(np.float64)
        if not per_key:
            a = np.repeat(a[:, :, None], dk, axis=2)
        gamma = np.cumprod(a[:, 0, :], axis=0)                  # [T, dk]
        kk, qq, vv = (x[:, 0].astype(np.float64) for x in (k, q, v))
        expect = np.zeros((T, dv))
        for t in range(T):
            for i in range(t + 1):
                expect[t] += vv[i] * np.dot(kk[i] * gamma[t] / gamma[i], qq[t])
        np.testing.assert_allclose(o[:, 0], expect, rtol=1e-12, atol=1e-13)
        if alpha_one:   # the state is the plain sum of outer products
            np.testing.assert_allclose(fin[0, 0], vv.T @ kk, rtol=1e-13, atol=1e-14)


def test_channel_uniform_gate_equals_scalar():
    rng = np.random.default_rng(4)
    T, H, dk, dv = 50, 3, 8, 8
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, per_key=0)
    alpha_pk = np.repeat(alpha[:, :, None], dk, axis=2)
    a = oracle.run(q, k, v, alpha, beta, [0, 20, T], np.concatenate([s0, s0]), interval=10)
    b = oracle.run(q, k, v, alpha_pk, beta, [0, 20, T], np.concatenate([s0, s0]), interval=10)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("beta_val", [0.0, 0.3, 1.0])
def test_fixed_point_state_already_maps_key(beta_val):
    """alpha=1, S0 = v k^T with |k| = 1: the token (k, v) changes nothing."""
    dk, dv = 64, 7
    rng = np.random.default_rng(5)
    Hm = np.array([[1.0]])
    while Hm.shape[0] < dk:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    kvec = (Hm[13] / 8.0).astype(np.float32)
    vvec = (np.round(rng.standard_normal(dv) * 4) / 4).astype(np.float32)
    s0 = np.outer(vvec, kvec).astype(np.float32)[None, None]
    k = kvec[None, None, :]
    v = vvec[None, None, :]
    q = rng.standard_normal((1, 1, dk)).astype(np.float32)
    alpha = np.ones((1, 1), np.float32)
    beta = np.full((1, 1), beta_val, np.float32)
    _, fin, _ = oracle.run(q, k, v, alpha, beta, [0, 1], s0)
    assert np.array_equal(fin, s0.astype(np.float64))


def test_pure_decay_matches_page_figures():
    """beta = 0, alpha = sigmoid(5) on every token: S_t = sigmoid(5)^t S0. The
    page prints sigma ~ 0.993 for the +5 bias and a decay product of order 1e-3
    over 950 tokens."""
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    bias = figs["sigmoid_of_alpha_bias"]["bias"]
    a32 = np.float32(1.0 / (1.0 + np.exp(-bias)))
    assert round(float(a32), figs["sigmoid_of_alpha_bias"]["printed_digits"]) == \
        figs["sigmoid_of_alpha_bias"]["value"]
    n = figs["decay_product_950_tokens"]["tokens"]
    T, H, dk, dv = n, 1, 4, 3
    rng = np.random.default_rng(6)
    s0 = rng.standard_normal((1, H, dv, dk)).astype(np.float32)
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    for per_key in (0, 1):
        alpha = np.full((T, H, dk) if per_key else (T, H), a32, np.float32)
        beta = np.zeros((T, H), np.float32)
        _, fin, snaps = oracle.run(q, k, v, alpha, beta, [0, T], s0, interval=50)
        factor = float(a32) ** n
        np.testing.assert_allclose(fin, factor * s0.astype(np.float64), rtol=1e-12)
        # every 50 tokens (crossing many chunk-sized spans) the factor is a32^(50 m)
        for m in range(1, T // 50 + 1):
            np.testing.assert_allclose(snaps[m - 1], float(a32) ** (50 * m) * s0[0].astype(np.float64), rtol=1e-12)
        order = figs["decay_product_950_tokens"]["order_of_magnitude"]
        assert order / 10 ** 0.5 < factor < order * 10 ** 0.5


def _encode_v(seq, pos):
    # three small integers, exact in bf16 (<= 256)
    return np.array([seq, pos % 128, pos // 128], np.float32)


def test_snapshot_placement_and_indexing_exact():
    """alpha = beta = 1 with one-hot keys k_t = e_{t mod d_k}: each token
    overwrites column (t mod d_k) of S with v_t, so every state column names the
    (sequence, position) of the token that wrote it. All arithmetic is exact."""
    dk, dv, H = 16, 3, 2
    lens = [37, 0, 64, 5, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    interval = 16
    k = np.zeros((T, H, dk), np.float32)
    q = np.zeros((T, H, dk), np.float32)
    v = np.zeros((T, H, dv), np.float32)
    for n, L in enumerate(lens):
        for p in range(L):
            t = cu[n] + p
            k[t, :, p % dk] = 1.0
            q[t, :, (3 * p) % dk] = 1.0
            v[t, :, :] = _encode_v(n + 1, p)
    alpha = np.ones((T, H), np.float32)
    beta = np.ones((T, H), np.float32)
    o, fin, snaps = oracle.run(bf16_bits(q), bf16_bits(k), bf16_bits(v), alpha, beta, cu,
                               interval=interval)
    assert snaps.shape[0] == sum(L // interval for L in lens)

    def expected_state(n, upto):
        S = np.zeros((dv, dk))
        for p in range(upto):
            S[:, p % dk] = _encode_v(n + 1, p)
        return S

    slot = 0
    for n, L in enumerate(lens):
        for m in range(1, L // interval + 1):
            for h in range(H):
                assert np.array_equal(snaps[slot, h], expected_state(n, m * interval)), (n, m)
            slot += 1
        for h in range(H):
            assert np.array_equal(fin[n, h], expected_state(n, L))
        for p in range(L):
            S = expected_state(n, p + 1)
            assert np.array_equal(o[cu[n] + p, 0], S[:, (3 * p) % dk])


def test_packing_equals_solo_runs():
    rng = np.random.default_rng(7)
    lens = [9, 0, 23, 1, 16]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, dk, dv = int(cu[-1]), 2, 8, 6
    for per_key in (0, 1):
        q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, per_key, n_seqs=len(lens))
        o, fin, snaps = oracle.run(q, k, v, alpha, beta, cu, s0, interval=4)
        slot = 0
        for n, L in enumerate(lens):
            sl = slice(cu[n], cu[n + 1])
            o1, f1, s1 = oracle.run(q[sl], k[sl], v[sl], alpha[sl], beta[sl], [0, L], s0[n:n + 1],
                                    interval=4)
            assert np.array_equal(o[sl], o1)
            assert np.array_equal(fin[n:n + 1], f1)
            assert np.array_equal(snaps[slot:slot + s1.shape[0]], s1)
            slot += s1.shape[0]


def test_prefix_reuse_from_snapshot():
    rng = np.random.default_rng(8)
    T, H, dk, dv, N = 100, 2, 8, 8, 48
    for per_key in (0, 1):
        q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, per_key)
        o, fin, snaps = oracle.run(q, k, v, alpha, beta, [0, T], s0, interval=N)
        o1, f1, _ = oracle.run(q[:N], k[:N], v[:N], alpha[:N], beta[:N], [0, N], s0)
        assert np.array_equal(snaps[0], f1[0])
        o2, f2, _ = oracle.run(q[N:], k[N:], v[N:], alpha[N:], beta[N:], [0, T - N],
                               f1.astype(np.float32))
        # the resumed run starts from the fp32-rounded snapshot: equal to rounding
        np.testing.assert_allclose(o2, o[N:], rtol=0, atol=1e-6 * np.abs(o).max())
        np.testing.assert_allclose(f2, fin, rtol=0, atol=1e-6 * np.abs(fin).max())
        assert np.array_equal(o1, o[:N])


def _literal_form(q, k, v, a, beta, S0):
    """S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and
    o_t = S_t q_t, evaluated as written with exact rationals."""
    T, dk, dv = len(q), len(q[0]), len(v[0])
    S = [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        M = [[(Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j]
              for j in range(dk)] for i in range(dk)]
        SD = [[S[r][c] * a[t][c] for c in range(dk)] for r in range(dv)]
        S = [[sum(SD[r][m] * M[m][c] for m in range(dk)) + beta[t] * v[t][r] * k[t][c]
              for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * q[t][c] for c in range(dk)) for r in range(dv)])
    return outs, S


@pytest.mark.parametrize("per_key", [0, 1])
def test_literal_product_form_exact_rationals(per_key):
    rng = np.random.default_rng(9)
    T, dk, dv = 5, 3, 2

    def dy(shape, scale):  # dyadic rationals, exact in fp32
        return (np.round(rng.uniform(-1, 1, size=shape) * scale) / scale).astype(np.float32)

    q, k, v = dy((T, dk), 64), dy((T, dk), 64), dy((T, dv), 64)
    beta = (np.round(rng.uniform(0, 1, size=T) * 64) / 64).astype(np.float32)
    if per_key:
        a = (np.round(rng.uniform(0.5, 1, size=(T, dk)) * 64) / 64).astype(np.float32)
    else:
        a1 = (np.round(rng.uniform(0.5, 1, size=T) * 64) / 64).astype(np.float32)
        a = np.repeat(a1[:, None], dk, axis=1)
    S0 = dy((dv, dk), 64)
    F = lambda arr: [[Fraction(float(x)) for x in row] for row in arr]  # noqa: E731
    outs, S = _literal_form(F(q), F(k), F(v), F(a), [Fraction(float(b)) for b in beta], F(S0))
    alpha = a[:, None, :] if per_key else a[:, :1]
    o, fin, _ = oracle.run(q[:, None], k[:, None], v[:, None], alpha, beta[:, None], [0, T],
                           S0[None, None])
    np.testing.assert_allclose(o[:, 0], np.array(outs, dtype=np.float64), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(fin[0, 0], np.array(S, dtype=np.float64), rtol=1e-14, atol=1e-15)


def test_state_size_figures():
    """State is d_v x d_k fp32 per head; the page-1 and page-2 figures follow."""
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    d = figs["state_values_per_head_d128"]["d"]
    assert d * d == figs["state_values_per_head_d128"]["value"]
    per_tok = figs["softmax_cache_values_per_token_head_d128"]["value"]
    assert d * d // per_tok == figs["crossover_tokens"]["value"]
    r = figs["ratio_at_262k"]
    assert r["tokens"] * per_tok // (d * d) == r["value"]
    g = figs["graft_cache_bytes_at_65536"]
    const = g["value"] - g["bytes_per_token"] * g["tokens"]
    assert round(const / 2 ** 20, 2) == g["constant_mib_printed"]
    m = figs["graft_model_state_shape"]
    state_bytes = m["kda_layers"] * m["heads"] * m["head_dim"] ** 2 * m["state_bytes_per_value"]
    assert state_bytes <= const   # the recurrent state is the bulk of the constant
    assert state_bytes / const > 0.9


def test_rejects_bad_inputs():
    rng = np.random.default_rng(10)
    T, H, dk, dv = 6, 1, 4, 4
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, 0)
    bad = alpha.copy(); bad[2, 0] = 0.0
    with pytest.raises(ValueError):
        oracle.run(q, k, v, bad, beta, [0, T])
    bad = alpha.copy(); bad[2, 0] = 1.5
    with pytest.raises(ValueError):
        oracle.run(q, k, v, bad, beta, [0, T])
    badb = beta.copy(); badb[0, 0] = -0.1
    with pytest.raises(ValueError):
        oracle.run(q, k, v, alpha, badb, [0, T])
    with pytest.raises(ValueError):
        oracle.run(q, k, v, alpha, beta, np.array([0, 4, 3, T]))


def test_ref_check_flags_corruption_and_nonfinite():
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, 1)
    o, fin, snaps = oracle.run(q, k, v, alpha, beta, [0, T], s0, interval=8)
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, [0, T], s0, 8, o, fin, snaps)
    assert rc == oracle.OK and rep["o_rel"] < 1e-6 and rep["n_snap"] == 5
    o_bad = o.astype(np.float32).copy(); o_bad[17, 1, 3] += 0.01 * np.abs(o).max()
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, [0, T], s0, 8, o_bad, fin, snaps)
    assert rc == oracle.MISMATCH and rep["o_rel"] > 5e-3
    s_bad = snaps.astype(np.float32).copy(); s_bad[3, 0, 2, 2] = np.nan
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, [0, T], s0, 8, o, fin, s_bad)
    assert rc == oracle.MISMATCH and rep["nonfinite"] == 1


def test_ref_check_normalises_each_slice():
    """The tolerance is relative to each (sequence, head) slice's own largest
    reference value (reading R13 of the comparison): a head 1000 times larger
    than another must not hide a 1 % error in the small one. The large slice
    comes first (head 0, sequence 0), so a normaliser carried over from an
    earlier slice, or taken over the whole tensor, passes what must fail."""
    rng = np.random.default_rng(13)
    lens = [48, 40]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, dk, dv = int(cu[-1]), 2, 8, 8
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, 1, n_seqs=2)
    v[:, 0] *= 1000.0
    s0[:, 0] *= 1000.0
    s0[0] *= 1000.0
    v[cu[0]:cu[1]] *= 1000.0
    o, fin, snaps = oracle.run(q, k, v, alpha, beta, cu, s0, interval=8)
    assert np.abs(o[:, 0]).max() > 300 * np.abs(o[cu[1]:, 1]).max()
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, cu, s0, 8, o, fin, snaps)
    assert rc == oracle.OK

    def planted(ref, idx, small):
        x = ref.astype(np.float32).copy()
        x[idx] += np.float32(0.01 * np.abs(small).max())
        return x

    # o: sequence 1, head 1 (the small slice)
    o_bad = planted(o, (cu[1] + 7, 1, 3), o[cu[1]:, 1])
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, cu, s0, 8, o_bad, fin, snaps)
    assert rc == oracle.MISMATCH and 0.005 < rep["o_rel"] < 0.02, rep
    # final state and a snapshot of sequence 1, head 1
    f_bad = planted(fin, (1, 1, 2, 5), fin[1, 1])
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, cu, s0, 8, o, f_bad, snaps)
    assert rc == oracle.MISMATCH and 0.005 < rep["final_rel"] < 0.02, rep
    n0 = lens[0] // 8
    s_bad = planted(snaps, (n0 + 2, 1, 4, 1), snaps[n0 + 2, 1])
    rc, rep = oracle.ref_check(q, k, v, alpha, beta, cu, s0, 8, o, fin, s_bad)
    assert rc == oracle.MISMATCH and 0.005 < rep["snap_rel"] < 0.02, rep


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(12)
    lens = [70, 3, 40]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, dk, dv = int(cu[-1]), 3, 16, 16
    q, k, v, alpha, beta, s0 = rand_inputs(rng, T, H, dk, dv, 1, n_seqs=3)
    a = oracle.run(q, k, v, alpha, beta, cu, s0, interval=16, threads=1)
    b = oracle.run(q, k, v, alpha, beta, cu, s0, interval=16, threads=8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
