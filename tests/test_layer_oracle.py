"""Pins of the layer front/back-end oracle (oracle/layer.py) against library
routines, closed forms, the page's gate figure and brute-force properties."""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import layer as L

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def test_conv_equals_numpy_convolve_per_channel():
    """Within one sequence and with zero state, each channel is the causal
    part of np.convolve with the reversed taps."""
    rng = np.random.default_rng(1)
    T, C = 37, 5
    x = _rand(rng, T, C)
    w = _rand(rng, C, 4)
    y, _ = L.conv4(x, w, [0, T])
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:T]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


def test_identity_and_shift_taps():
    rng = np.random.default_rng(2)
    T, C = 9, 3
    x = _rand(rng, T, C)
    state = _rand(rng, 1, 3, C)
    y, st = L.conv4(x, np.tile([0.0, 0.0, 0.0, 1.0], (C, 1)), [0, T], state)
    np.testing.assert_array_equal(y, x)                         # identity tap
    y1, _ = L.conv4(x, np.tile([0.0, 0.0, 1.0, 0.0], (C, 1)), [0, T], state)
    np.testing.assert_array_equal(y1[1:], x[:-1])                # one token back
    np.testing.assert_array_equal(y1[0], state[0, 2])            # the newest carried input
    y3, _ = L.conv4(x, np.tile([1.0, 0.0, 0.0, 0.0], (C, 1)), [0, T], state)
    np.testing.assert_array_equal(y3[:3], state[0])              # oldest first
    np.testing.assert_array_equal(st[0], x[-3:])


def test_causal_and_sequence_local():
    rng = np.random.default_rng(3)
    cu = [0, 10, 10, 13, 30]
    T, C = cu[-1], 4
    x = _rand(rng, T, C)
    w = _rand(rng, C, 4)
    y, st = L.conv4(x, w, cu)
    for t in (5, 12, 20):
        x2 = x.copy()
        x2[t] += 1.0
        y2, _ = L.conv4(x2, w, cu)
        np.testing.assert_array_equal(y2[:t], y[:t])             # nothing before t changes
        seq = np.searchsorted(cu, t, side="right") - 1
        end = cu[seq + 1]
        np.testing.assert_array_equal(y2[end:], y[end:])         # nor any later sequence
    for n in range(len(cu) - 1):                                  # packed == solo
        ys, sts = L.conv4(x[cu[n]:cu[n + 1]], w, [0, cu[n + 1] - cu[n]])
        np.testing.assert_array_equal(ys, y[cu[n]:cu[n + 1]])
        np.testing.assert_array_equal(sts[0], st[n])


def test_state_handoff_equals_unsplit():
    rng = np.random.default_rng(4)
    T, H, d = 23, 2, 8
    xs = [_rand(rng, T, H, d) for _ in range(3)]
    w = _rand(rng, 3, H, d, 4)
    al, bl = _rand(rng, T, H), _rand(rng, T, H)
    full = L.layer_front(*xs, w, [0, T], None, al, 5.0, bl)
    for a in (1, 2, 3, 11):
        p1 = L.layer_front(*[x[:a] for x in xs], w, [0, a], None, al[:a], 5.0, bl[:a])
        p2 = L.layer_front(*[x[a:] for x in xs], w, [0, T - a], p1[5], al[a:], 5.0, bl[a:])
        for i in range(5):
            np.testing.assert_allclose(np.concatenate([p1[i], p2[i]]), full[i], rtol=0, atol=1e-14)
        np.testing.assert_array_equal(p2[5], full[5])


def test_short_sequence_state_shifts_in():
    rng = np.random.default_rng(5)
    C = 3
    state = _rand(rng, 1, 3, C)
    x = _rand(rng, 2, C)
    _, st = L.conv4(x, _rand(rng, C, 4), [0, 2], state)
    np.testing.assert_array_equal(st[0, 0], state[0, 2])
    np.testing.assert_array_equal(st[0, 1:], x)


def test_gates_and_normalisation():
    fig = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))
    rng = np.random.default_rng(6)
    T, H, d = 7, 3, 16
    xs = [_rand(rng, T, H, d) for _ in range(3)]
    w = np.zeros((3, H, d, 4))
    w[..., 3] = 1.0                                               # identity taps
    q, k, v, a, b, _ = L.layer_front(*xs, w, [0, T], None, np.zeros((T, H)), 5.0, _rand(rng, T, H))
    # the page's gate: bias +5 gives sigmoid(5) ~ 0.993
    g = fig["sigmoid_of_alpha_bias"]
    assert abs(a[0, 0] - g["value"]) < 0.5 * 10.0 ** -g["printed_digits"]
    np.testing.assert_allclose(a, expit(5.0), rtol=1e-15)
    np.testing.assert_allclose(v, xs[2] * expit(xs[2]), rtol=1e-14)          # identity conv, SiLU
    np.testing.assert_allclose(np.sum(q * q, axis=-1), 1.0, atol=1e-6)        # unit rows (to eps)
    s = xs[0] * expit(xs[0])
    np.testing.assert_allclose(q, s / np.linalg.norm(s, axis=-1, keepdims=True), rtol=1e-6)


def test_back_end_rmsnorm_gate():
    rng = np.random.default_rng(7)
    T, H, dv = 5, 2, 32
    o = _rand(rng, T, H, dv, scale=3.0)
    wn = rng.uniform(0.5, 1.5, dv)
    big = np.full((T, H, dv), 60.0)                               # sigmoid = 1 in fp64
    y = L.layer_back(o, big, np.ones(dv), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(L.layer_back(7.0 * o, big, wn, 0.0), L.layer_back(o, big, wn, 0.0), rtol=1e-13)
    half = L.layer_back(o, np.zeros((T, H, dv)), wn, 0.0)
    np.testing.assert_allclose(half, 0.5 * L.layer_back(o, big, wn, 0.0), rtol=1e-13)


def test_carried_conv_state_matches_page_memory_constant():
    """The page's cache constant (205 745 664 B at L = 65 536 with 3 072 B per
    token, section '1. Память') minus the recurrent states of its 18 KDA layers
    (14 heads x 64 x 64 fp32 each) leaves 290 304 B: exactly one carried
    convolution state per layer as laid out here (3 taps x q, k, v x 14 heads
    x 64 channels) stored in bf16."""
    fig = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))["graft_cache_bytes_at_65536"]
    constant = fig["value"] - fig["bytes_per_token"] * fig["tokens"]
    layers, H, d = 18, 14, 64
    state_bytes = layers * H * d * d * 4
    rng = np.random.default_rng(8)
    T = 5
    xs = [_rand(rng, T, H, d) for _ in range(3)]
    *_, conv_state = L.layer_front(*xs, _rand(rng, 3, H, d, 4), [0, T], None, _rand(rng, T, H), 5.0,
                                   _rand(rng, T, H))
    assert conv_state.shape == (1, 3, 3, H, d)
    assert constant - state_bytes == layers * conv_state[0].size * 2
