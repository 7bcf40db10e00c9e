"""GPU parity of the backward pass (kda_prefill_backward) against the fp64
oracle's token-by-token backward (kda_oracle_backward), through the C ABI.

Tolerance: every gradient within 2e-3 of the oracle as the slice-max relative
error (max |x - r| / max |r| per (sequence, head) slice), the measure used for
the forward; fp32 arithmetic on the chunked form, against fp64.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_72_amd as kda
import oracle
from gated_delta_rule_72_amd import workloads as wl

from gpu_util import custom, device

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-3
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial")


def _grads_in(w, dev, seed, with_final=True):
    inp = wl.make_prefill_inputs(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    d_o = torch.randn((w.T, w.H, w.dv), generator=g, device=dev, dtype=torch.float32)
    d_f = (torch.randn((w.num_seqs, w.H, w.dv, w.dk), generator=g, device=dev, dtype=torch.float32)
           if with_final else None)
    return inp, d_o, d_f


def _slice_err(x, r, cu, per_token=True):
    worst = 0.0
    if not per_token:                                   # [N, H, ...]
        for n in range(x.shape[0]):
            for h in range(x.shape[1]):
                den = max(np.max(np.abs(r[n, h])), 1e-30)
                worst = max(worst, np.max(np.abs(x[n, h] - r[n, h])) / den)
        return worst
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        if e == s:
            continue
        for h in range(x.shape[1]):
            den = max(np.max(np.abs(r[s:e, h])), 1e-30)
            worst = max(worst, np.max(np.abs(x[s:e, h] - r[s:e, h])) / den)
    return worst


def _check(inp, d_o, d_f, got, heads=None, tol=GRAD_TOL):
    H = inp["q"].shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else t.index_select(1, torch.tensor(hs, device=t.device))  # noqa: E731
    A = {n: wl.to_oracle_arrays(sel(inp[n])) for n in ("q", "k", "v", "alpha", "beta")}
    init = None if inp["initial_state"] is None else sel(inp["initial_state"]).cpu().numpy()
    cu = inp["cu_seqlens_host"].numpy()
    ref = oracle.backward(A["q"], A["k"], A["v"], A["alpha"], A["beta"], cu, init,
                          sel(d_o).cpu().numpy(), None if d_f is None else sel(d_f).cpu().numpy())
    errs = {}
    for name, x in zip(NAMES, got):
        xs = sel(x).cpu().numpy().astype(np.float64)
        errs[name] = _slice_err(xs, ref[name], cu, per_token=name != "d_initial")
    print("backward errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= tol, (name, e)
    return errs


def _run(inp, d_o, d_f, want_init=True):
    out = kda.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], d_o, inp["cu_seqlens"],
                               inp["initial_state"], d_f, cu_seqlens_host=inp["cu_seqlens_host"],
                               want_d_initial=want_init)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_small_varlen(d, gate, dtype):
    w = custom(f"bwd_{d}_{gate}_{dtype}", H=2, d=d, lens=(200, 1, 0, 64, 129, 63), gate=gate, dtype=dtype,
               s0_std=0.05, seed=70)
    inp, d_o, d_f = _grads_in(w, device(), seed=71)
    _check(inp, d_o, d_f, _run(inp, d_o, d_f))


@pytest.mark.parametrize("d,gate", [(64, "per_key"), (128, "scalar"), (128, "per_key")])
def test_backward_segmented_scan(d, gate):
    """Sequences of 18 and 10 chunks with few heads: the state-gradient scan is
    cut into segments (maps, a scan over segments, then each segment again)."""
    w = custom(f"bwd_seg_{d}_{gate}", H=2, d=d, lens=(1100, 600, 3, 0), gate=gate, s0_std=0.05, seed=79)
    inp, d_o, d_f = _grads_in(w, device(), seed=80)
    _check(inp, d_o, d_f, _run(inp, d_o, d_f))


def test_backward_without_initial_or_final_state():
    w = custom("bwd_zero_states", H=2, d=64, lens=(150, 70), gate="per_key", s0_std=0.0, seed=72)
    inp, d_o, _ = _grads_in(w, device(), seed=73, with_final=False)
    inp["initial_state"] = None
    got = _run(inp, d_o, None)
    _check(inp, d_o, None, got)


def test_backward_only_final_gradient_and_empty_sequences():
    """d_o = 0: every gradient comes through the final state; empty sequences
    hand d_final straight to d_initial."""
    w = custom("bwd_final_only", H=2, d=64, lens=(0, 130, 0), gate="scalar", s0_std=0.05, seed=74)
    inp, d_o, d_f = _grads_in(w, device(), seed=75)
    d_o.zero_()
    got = _run(inp, d_o, d_f)
    assert torch.equal(got[5][0], d_f[0]) and torch.equal(got[5][2], d_f[2])
    _check(inp, d_o, d_f, got)


def test_backward_all_sequences_empty():
    """T = 0 with two (empty) sequences: no token gradients, and d_initial is
    d_final bit for bit (zero when d_final is not given)."""
    dev = device()
    H, d = 2, 64
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)  # noqa: E731
    q = torch.zeros((0, H, d), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 0, 0], dtype=torch.int64, device=dev)
    d_f = torch.randn((2, H, d, d), device=dev)
    out = kda.prefill_backward(q, q, q, z(0, H, d), z(0, H), z(0, H, d), cu, None, d_f)
    torch.cuda.synchronize()
    assert all(x.numel() == 0 for x in out[:5])
    assert torch.equal(out[5], d_f)
    out = kda.prefill_backward(q, q, q, z(0, H, d), z(0, H), z(0, H, d), cu, None, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[5]) == 0


def test_backward_deterministic():
    w = custom("bwd_det", H=2, d=128, lens=(300, 5), gate="per_key", seed=76)
    inp, d_o, d_f = _grads_in(w, device(), seed=77)
    a = _run(inp, d_o, d_f)
    b = _run(inp, d_o, d_f)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_kda_layer_shape():
    """The KDA-layer workload (T=8192, H=14, d=64, per-key gate) at full size,
    all heads against the oracle."""
    w = wl.KDA_LAYER
    inp, d_o, d_f = _grads_in(w, device(), seed=78)
    got = _run(inp, d_o, d_f)
    _check(inp, d_o, d_f, got)


@pytest.mark.parametrize("group", range(2))
def test_backward_long_prefill_full_size(group):
    """The long-prefill workload (T=262144, H=16, d=128, scalar gate) at full
    size in the benchmark's launch configuration (automatic segment plans for
    the forward recompute and the state-gradient scan); 8 of the 16 heads per
    case against the oracle, all heads over the two cases (about 40 s of host
    time, one thread per head)."""
    w = wl.LONG_PREFILL
    inp, d_o, d_f = _grads_in(w, device(), seed=81)
    got = _run(inp, d_o, d_f)
    print(f"long-prefill backward heads {8 * group}..{8 * group + 7}", flush=True)
    _check(inp, d_o, d_f, got, heads=range(8 * group, 8 * group + 8))


def test_backward_d_initial_may_be_d_final():
    """d_initial_state written over the d_final_state buffer, on the shape
    whose state-gradient scan is cut into segments: every gradient equals the
    run with separate buffers bit for bit, and the oracle's."""
    w = custom("bwd_alias", H=2, d=64, lens=(1100, 600, 3, 0), gate="per_key", s0_std=0.05, seed=84)
    inp, d_o, d_f = _grads_in(w, device(), seed=85)
    ref = _run(inp, d_o, d_f)
    buf = d_f.clone()
    T, H, d = w.T, w.H, w.dk
    f32 = dict(dtype=torch.float32, device=d_o.device)
    dq, dk, dv = torch.empty((T, H, d), **f32), torch.empty((T, H, d), **f32), torch.empty((T, H, d), **f32)
    da, db = torch.empty(inp["alpha"].shape, **f32), torch.empty((T, H), **f32)
    shape = kda.make_shape(H, d, d, inp["q"].dtype, True)
    ws = torch.empty(kda.kda_prefill_backward_workspace_size(shape, inp["cu_seqlens_host"]), dtype=torch.uint8,
                     device=d_o.device)
    kda.kda_prefill_backward(shape, inp["cu_seqlens_host"], inp["cu_seqlens"], inp["q"], inp["k"], inp["v"],
                             inp["alpha"], inp["beta"], inp["initial_state"], d_o, buf, dq, dk, dv, da, db, buf, ws)
    torch.cuda.synchronize()
    for x, r in zip((dq, dk, dv, da, db, buf), ref):
        assert torch.equal(x, r)
    _check(inp, d_o, d_f, (dq, dk, dv, da, db, buf))


def _abi_backward(inp, d_o, d_final, d_initial):
    """kda_prefill_backward through the C ABI with caller-chosen d_final and
    d_initial buffers (they may be one buffer)."""
    T, H, dk = inp["q"].shape
    dv = inp["v"].shape[2]
    f32 = dict(dtype=torch.float32, device=d_o.device)
    dq, dk_, dv_ = torch.empty((T, H, dk), **f32), torch.empty((T, H, dk), **f32), torch.empty((T, H, dv), **f32)
    da, db = torch.empty(inp["alpha"].shape, **f32), torch.empty((T, H), **f32)
    shape = kda.make_shape(H, dk, dv, inp["q"].dtype, inp["alpha"].dim() == 3)
    ws = torch.empty(kda.kda_prefill_backward_workspace_size(shape, inp["cu_seqlens_host"]), dtype=torch.uint8,
                     device=d_o.device)
    kda.kda_prefill_backward(shape, inp["cu_seqlens_host"], inp["cu_seqlens"], inp["q"], inp["k"], inp["v"],
                             inp["alpha"], inp["beta"], inp["initial_state"], d_o, d_final, dq, dk_, dv_, da, db,
                             d_initial, ws)
    torch.cuda.synchronize()
    return (dq, dk_, dv_, da, db, d_initial), ws.numel()


@pytest.mark.parametrize("H,d,gate,dtype", [(5, 64, "per_key", "bf16"), (3, 128, "scalar", "fp32")])
@pytest.mark.parametrize("budget", ["one_head", "below_full"])
def test_backward_in_head_groups(H, d, gate, dtype, budget, monkeypatch):
    """A workspace budget below what all heads need at once runs the heads in
    groups (inputs gathered per group into the workspace, gradients scattered
    back), here one head per group or groups of ceil(H/2) with a smaller last
    group, on the shape whose state-gradient scan is cut into segments: a
    smaller workspace, every gradient against the oracle, and d_initial
    written over d_final equal bit for bit to separate buffers."""
    w = custom(f"bwd_groups_{H}_{d}_{gate}", H=H, d=d, lens=(1100, 600, 3, 0), gate=gate, dtype=dtype,
               s0_std=0.05, seed=88)
    inp, d_o, d_f = _grads_in(w, device(), seed=89)
    _, full = _abi_backward(inp, d_o, d_f, torch.empty_like(d_f))
    monkeypatch.setenv("KDA_BACKWARD_BUDGET_BYTES", "1" if budget == "one_head" else str(full - 1))
    got, grouped = _abi_backward(inp, d_o, d_f, torch.empty_like(d_f))
    print(f"workspace {full} -> {grouped} bytes", flush=True)
    assert grouped < full
    _check(inp, d_o, d_f, got)
    buf = d_f.clone()
    alias, _ = _abi_backward(inp, d_o, buf, buf)
    for x, r in zip(alias, got):
        assert torch.equal(x, r)


def test_backward_varlen_full_size():
    """The varlen workload (32 packed sequences of U[1024, 32768] tokens, H=32,
    d=128, per-key gate, initial states) at full size in the benchmark's
    launch configuration; heads 0-3 and 28-31 against the oracle (about a
    minute of host time, one thread per head)."""
    w = wl.VARLEN
    inp, d_o, d_f = _grads_in(w, device(), seed=92)
    got = _run(inp, d_o, d_f)
    _check(inp, d_o, d_f, got, heads=(0, 1, 2, 3, 28, 29, 30, 31))


def test_backward_per_key_decay_at_the_limit():
    """Key channels whose decay over every 32 tokens is 2^-119.5, just inside
    the backward's stated limit of 2^-120 (decay factors relative to a chunk's
    middle row): every gradient within tolerance of the oracle."""
    w = custom("bwd_pk_limit", H=2, d=128, lens=(300, 81, 16), gate="per_key", s0_std=0.05, seed=86)
    inp, d_o, d_f = _grads_in(w, device(), seed=87)
    a = inp["alpha"].clone()
    a[:, :, :8] = 2.0 ** (-119.5 / 32)
    inp["alpha"] = a
    _check(inp, d_o, d_f, _run(inp, d_o, d_f))


def test_autograd_function_routes_gradients():
    """gated_delta_rule (torch.autograd glue): loss.backward() gives exactly
    what kda.prefill_backward gives for the same incoming gradients."""
    w = custom("bwd_autograd", H=2, d=64, lens=(150, 30), gate="per_key", dtype="fp32", s0_std=0.05, seed=82)
    inp, d_o, d_f = _grads_in(w, device(), seed=83)
    leaves = {n: inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "alpha", "beta", "initial_state")}
    o, fin = kda.gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["alpha"], leaves["beta"],
                                  inp["cu_seqlens"], leaves["initial_state"], inp["cu_seqlens_host"])
    ((o * d_o).sum() + (fin * d_f).sum()).backward()
    torch.cuda.synchronize()
    ref = _run(inp, d_o, d_f)
    for (n, x), r in zip(leaves.items(), ref):
        assert torch.equal(x.grad, r), n
