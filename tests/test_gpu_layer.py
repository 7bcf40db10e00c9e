"""GPU parity of the KDA layer front and back end (kda_layer_front,
kda_layer_back) against the fp64 oracle in oracle/layer.py, through the C ABI.

Tolerances (max error over a (sequence, head) slice relative to the slice's
max |reference|): bf16 outputs 4e-3 (one bf16 rounding is 2^-9), fp32 outputs
2e-5; gates 1e-5 absolute; the carried conv state is a copy, checked bit for
bit.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_72_amd as kda
from gated_delta_rule_72_amd import workloads as wl
from oracle import layer as L

from gpu_util import check_prefill, custom, device

pytestmark = pytest.mark.gpu


def _np(t):
    return None if t is None else wl.to_oracle_arrays(t)


def _rel(x, ref, cu=None):
    x = x.astype(np.float64)
    if not np.all(np.isfinite(x)) or not np.all(np.isfinite(ref)):
        bad = np.argwhere(~np.isfinite(x))
        print(f"non-finite: candidate {len(bad)} (first {bad[:4].tolist()}), "
              f"reference {int(np.sum(~np.isfinite(ref)))}", flush=True)
    if cu is None:
        return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30)
    worst = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(ref.shape[1]):
            r = ref[s:e, h]
            if r.size:
                worst = max(worst, np.max(np.abs(x[s:e, h] - r)) / max(np.max(np.abs(r)), 1e-30))
    return worst


def _front(li, bias=5.0, state=True):
    return kda.layer_front(li["xq"], li["xk"], li["xv"], li["conv_w"], li["alpha_logit"], li["beta_logit"],
                           li["cu_seqlens"], li["conv_state"] if state else None, bias,
                           cu_seqlens_host=li["cu_seqlens_host"])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_front_matches_oracle(d, gate, dtype):
    w = custom(f"front_{d}_{gate}_{dtype}", H=3, d=d, lens=(70, 1, 0, 2, 64, 129), gate=gate, dtype=dtype, seed=41)
    li = wl.make_layer_inputs(w, device())
    q, k, v, a, b, st = _front(li, bias=4.5)
    torch.cuda.synchronize()
    cu = li["cu_seqlens_host"].numpy()
    rq, rk, rv, ra, rb, rst = L.layer_front(_np(li["xq"]), _np(li["xk"]), _np(li["xv"]), _np(li["conv_w"]), cu,
                                            _np(li["conv_state"]), _np(li["alpha_logit"]), 4.5,
                                            _np(li["beta_logit"]))
    tol = 4e-3 if dtype == "bf16" else 2e-5
    for name, x, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        err = _rel(_np_f(x), r, cu)
        print(f"{name}: {err:.3e}", flush=True)
        assert err <= tol, (name, err)
    assert np.max(np.abs(a.cpu().numpy() - ra)) <= 1e-5
    assert np.max(np.abs(b.cpu().numpy() - rb)) <= 1e-5
    assert np.array_equal(_np_f(st), rst)                        # a copy of inputs: exact


def _np_f(t):
    """device tensor -> float64 numpy (bf16 exactly)."""
    return t.float().cpu().numpy().astype(np.float64)


def test_front_without_state_and_state_handoff_bitwise():
    w = custom("handoff", H=2, d=128, lens=(300,), gate="per_key", seed=42)
    li = wl.make_layer_inputs(w, device(), conv_state=False)
    full = _front(li, state=False)
    for a in (1, 2, 3, 64, 199):
        part = lambda s, e, stt: kda.layer_front(  # noqa: E731
            li["xq"][s:e].contiguous(), li["xk"][s:e].contiguous(), li["xv"][s:e].contiguous(), li["conv_w"],
            li["alpha_logit"][s:e].contiguous(), li["beta_logit"][s:e].contiguous(), conv_state=stt)
        p1 = part(0, a, None)
        p2 = part(a, 300, p1[5])
        torch.cuda.synchronize()
        for i in range(5):
            assert torch.equal(torch.cat([p1[i], p2[i]]), full[i]), (a, i)
        assert torch.equal(p2[5], full[5])


@pytest.mark.parametrize("gate", ["scalar", "per_key"])
def test_front_long_pack_matches_oracle(gate):
    """A pack past 32768 rows, where a workgroup takes 8-token tiles:
    sequence starts inside and at the edges of tiles, empty and one-token
    sequences, and a ragged last tile."""
    lens = (9000, 1, 0, 3, 17000, 2, 6813)       # T = 32819
    w = custom(f"front_long_{gate}", H=2, d=64, lens=lens, gate=gate, seed=44)
    li = wl.make_layer_inputs(w, device())
    q, k, v, a, b, st = _front(li)
    torch.cuda.synchronize()
    cu = li["cu_seqlens_host"].numpy()
    rq, rk, rv, ra, rb, rst = L.layer_front(_np(li["xq"]), _np(li["xk"]), _np(li["xv"]), _np(li["conv_w"]), cu,
                                            _np(li["conv_state"]), _np(li["alpha_logit"]), 5.0,
                                            _np(li["beta_logit"]))
    for name, x, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        err = _rel(_np_f(x), r, cu)
        print(f"{name}: {err:.3e}", flush=True)
        assert err <= 4e-3, (name, err)
    assert np.max(np.abs(a.cpu().numpy() - ra)) <= 1e-5
    assert np.max(np.abs(b.cpu().numpy() - rb)) <= 1e-5
    assert np.array_equal(_np_f(st), rst)


@pytest.mark.parametrize("gate", ["scalar", "per_key"])
def test_front_long_path_equals_short_path_bitwise(gate):
    """One sequence of 40013 rows takes the 8-token-tile launch; its two
    halves, each under 32768 rows and joined by the carried state, take the
    4-token-tile launch. Every output is the same bits."""
    w = custom(f"front_split_{gate}", H=2, d=128, lens=(40013,), gate=gate, seed=45)
    li = wl.make_layer_inputs(w, device())
    full = _front(li)
    T = 40013
    for a in (20000, 8195):
        part = lambda s, e, stt: kda.layer_front(  # noqa: E731
            li["xq"][s:e].contiguous(), li["xk"][s:e].contiguous(), li["xv"][s:e].contiguous(), li["conv_w"],
            li["alpha_logit"][s:e].contiguous(), li["beta_logit"][s:e].contiguous(), conv_state=stt)
        p1 = part(0, a, li["conv_state"])
        p2 = part(a, T, p1[5])
        torch.cuda.synchronize()
        for i in range(5):
            assert torch.equal(torch.cat([p1[i], p2[i]]), full[i]), (a, i)
        assert torch.equal(p2[5], full[5])


def test_front_all_sequences_empty_passes_state_through():
    dev = device()
    H, d = 2, 64
    x = torch.zeros((0, H, d), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 0, 0], dtype=torch.int64, device=dev)
    st = torch.randn((2, 3, 3, H, d), device=dev).to(torch.bfloat16)
    w = torch.zeros((3, H, d, 4), dtype=torch.float32, device=dev)
    z = torch.zeros((0, H), dtype=torch.float32, device=dev)
    q, k, v, a, b, st_out = kda.layer_front(x, x, x, w, z, z, cu, st)
    torch.cuda.synchronize()
    assert q.numel() == 0 and torch.equal(st_out, st)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_back_matches_oracle(d, out_dtype):
    w = custom(f"back_{d}", H=3, d=d, lens=(257,), seed=43)
    li = wl.make_layer_inputs(w, device())
    y = kda.layer_back(li["o"], li["g_logit"], li["norm_w"], 1e-6, out_dtype)
    torch.cuda.synchronize()
    ref = L.layer_back(_np(li["o"]), _np(li["g_logit"]), _np(li["norm_w"]), 1e-6)
    err = _rel(_np_f(y), ref, li["cu_seqlens_host"].numpy())
    print(f"back: {err:.3e}", flush=True)
    assert err <= (4e-3 if out_dtype == torch.bfloat16 else 2e-5)


def test_front_recurrence_back_end_to_end():
    """front -> kda_prefill_chunked -> back on a varlen pack, against the
    oracle's front, token recurrence and back end composed in fp64. fp32
    storage, so that no bf16 rounding of the front's outputs enters the
    recurrence's error budget (2e-3 on o; RMSNorm rescales it per token)."""
    import oracle
    w = custom("layer_e2e", H=2, d=64, lens=(150, 7, 64), gate="per_key", dtype="fp32", s0_std=0.02, seed=44)
    dev = device()
    li = wl.make_layer_inputs(w, dev)
    s0 = wl.make_prefill_inputs(w, dev)["initial_state"]
    q, k, v, a, b, _ = _front(li)
    o, fin, _ = kda.prefill_chunked(q, k, v, a, b, li["cu_seqlens"], s0, 0, cu_seqlens_host=li["cu_seqlens_host"])
    y = kda.layer_back(o, li["g_logit"], li["norm_w"], 1e-6, torch.float32)
    torch.cuda.synchronize()
    # the recurrence's own parity (against the oracle on the GPU front's outputs)
    inp = dict(q=q, k=k, v=v, alpha=a, beta=b, cu_seqlens=li["cu_seqlens"], cu_seqlens_host=li["cu_seqlens_host"],
               initial_state=s0)
    check_prefill(inp, (o, fin, None), 0)
    # and the whole layer against the fp64 composition
    cu = li["cu_seqlens_host"].numpy()
    rq, rk, rv, ra, rb, _ = L.layer_front(_np(li["xq"]), _np(li["xk"]), _np(li["xv"]), _np(li["conv_w"]), cu,
                                          _np(li["conv_state"]), _np(li["alpha_logit"]), 5.0, _np(li["beta_logit"]))
    f32 = lambda x: x.astype(np.float32)  # noqa: E731
    ro, _, _ = oracle.run(f32(rq), f32(rk), f32(rv), f32(ra), f32(rb), cu, s0.cpu().numpy(), 0)
    ref = L.layer_back(ro, _np(li["g_logit"]), _np(li["norm_w"]), 1e-6)
    err = _rel(_np_f(y), ref, cu)
    print(f"layer: {err:.3e}", flush=True)
    assert err <= 5e-3


def test_kda_layer_shape_full():
    """The KDA-layer workload shape (T=8192, H=14, d=64, per-key alpha): front
    and back against the oracle on every head."""
    w = wl.KDA_LAYER
    li = wl.make_layer_inputs(w, device())
    q, k, v, a, b, st = _front(li)
    y = kda.layer_back(li["o"], li["g_logit"], li["norm_w"], 1e-6, torch.bfloat16)
    torch.cuda.synchronize()
    cu = li["cu_seqlens_host"].numpy()
    rq, rk, rv, ra, rb, rst = L.layer_front(_np(li["xq"]), _np(li["xk"]), _np(li["xv"]), _np(li["conv_w"]), cu,
                                            _np(li["conv_state"]), _np(li["alpha_logit"]), 5.0,
                                            _np(li["beta_logit"]))
    for name, x, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert _rel(_np_f(x), r, cu) <= 4e-3, name
    assert np.max(np.abs(a.cpu().numpy() - ra)) <= 1e-5
    assert np.array_equal(_np_f(st), rst)
    ref = L.layer_back(_np(li["o"]), _np(li["g_logit"]), _np(li["norm_w"]), 1e-6)
    assert _rel(_np_f(y), ref, cu) <= 4e-3
