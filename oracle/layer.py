"""Front and back end of a KDA layer around the recurrence, in fp64 numpy.

TEST INFRASTRUCTURE: used only by tests/, never by the GPU library.

Page "kda-graft: Qwen2.5-0.5B с трансплантированным KDA" (ailist.pro), section
"Идея и архитектура": each KDA layer adds a 4-tap convolution initialised as
an identity tap, an alpha gate with bias +5 (sigmoid(5) ~ 0.993, the memory
barely forgets), beta, an output gate and RMSNorm. The page prints no formulas;
the readings taken here (each listed in the design notes) are:

  F2-R1  the convolution is causal and depthwise over the q, k and v channels
         (H * d each), 4 taps over the current and the 3 previous tokens of
         the same sequence; taps are stored oldest first, so the identity tap
         is [0, 0, 0, 1]; before a sequence's first token the taps read a
         carried convolution state (the 3 previous inputs) or zeros;
  F2-R2  SiLU follows the convolution (x * sigmoid(x));
  F2-R3  q and k are then L2-normalised over d per (token, head):
         x / sqrt(sum x^2 + 1e-6);
  F2-R4  alpha = sigmoid(alpha_logit + alpha_bias), beta = sigmoid(beta_logit);
  F2-R5  the output is RMSNorm over d_v per (token, head) with a learned
         weight, times a sigmoid output gate:
         o * rsqrt(mean(o^2) + eps) * w * sigmoid(g_logit);
  F2-R6  the carried state after a sequence holds its last 3 convolution
         inputs (oldest first), shifted in from the incoming state when the
         sequence is shorter than 3.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:          # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def conv4(x, w, cu, state=None):
    """Causal depthwise 4-tap convolution within each sequence.
    x [T, C]; w [C, 4] (taps oldest first); cu [N+1]; state [N, 3, C] or None.
    Returns (y [T, C], state_out [N, 3, C])."""
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    N = len(cu) - 1
    y = np.zeros((T, C))
    st_out = np.zeros((N, 3, C))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        prev = np.zeros((3, C)) if state is None else _f64(state[n])
        ext = np.concatenate([prev, x[s:e]], axis=0)          # [3 + len, C]
        for t in range(e - s):
            win = ext[t:t + 4]                                  # tokens t-3 .. t
            y[s + t] = np.sum(win * w.T, axis=0)
        st_out[n] = ext[-3:]
    return y, st_out


def layer_front(xq, xk, xv, conv_w, cu, conv_state=None, alpha_logit=None, alpha_bias=5.0,
                beta_logit=None):
    """xq, xk, xv [T, H, d]; conv_w [3, H, d, 4]; conv_state [N, 3, 3, H, d] or None
    (q, k, v; taps oldest first). Returns q, k, v [T,H,d], alpha, beta, state_out."""
    T, H, d = np.asarray(xq).shape
    outs, states = [], []
    for j, x in enumerate((xq, xk, xv)):
        st = None if conv_state is None else np.asarray(conv_state)[:, j].reshape(len(cu) - 1, 3, H * d)
        y, so = conv4(np.asarray(x).reshape(T, H * d), np.asarray(conv_w)[j].reshape(H * d, 4), cu, st)
        outs.append(silu(y).reshape(T, H, d))
        states.append(so.reshape(len(cu) - 1, 3, H, d))
    q, k, v = outs
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + L2_EPS)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + L2_EPS)
    alpha = sigmoid(_f64(alpha_logit) + alpha_bias)
    beta = sigmoid(_f64(beta_logit))
    return q, k, v, alpha, beta, np.stack(states, axis=1)


def layer_back(o, g_logit, norm_w, eps=1e-6):
    """o, g_logit [T, H, dv]; norm_w [dv]. RMSNorm over dv times sigmoid gate."""
    o = _f64(o)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * _f64(norm_w) * sigmoid(_f64(g_logit))
