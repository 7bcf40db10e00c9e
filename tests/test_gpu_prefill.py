"""GPU parity of kda_prefill_chunked against the fp64 CPU oracle (through the C ABI).

Tolerances: max relative error (slice-max normalised) 2e-3 on o and 1e-3 on
final states and snapshots; bit-exact for cu_seqlens indexing and snapshot
placement (exact-integer test).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_72_amd as kda
from gated_delta_rule_72_amd import workloads as wl

from gpu_util import check_prefill, custom, device, run_prefill

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_small_varlen(d, gate, dtype):
    dev = device()
    w = custom(f"small_{d}_{gate}_{dtype}", H=3, d=d, lens=(200, 1, 0, 64, 129, 63), gate=gate,
               dtype=dtype, interval=64, seed=11)
    print(f"case {w.name} lens={w.seq_lens}", flush=True)
    inp = wl.make_prefill_inputs(w, dev)
    outs = run_prefill(inp, w.interval)
    check_prefill(inp, outs, w.interval)


@pytest.mark.parametrize("gate", ["scalar", "per_key"])
def test_prefill_zero_initial_state_long(gate):
    dev = device()
    w = custom(f"long_{gate}", H=2, d=128, lens=(3000,), gate=gate, s0_std=0.0, seed=12,
               alpha_bias=4.0 if gate == "scalar" else 5.0)
    print(f"case {w.name}", flush=True)
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, 0), 0)


def test_tiny_recurrence_config():
    """B=1 H=1 d=64 T=256 fp32, scalar alpha, zero initial state."""
    dev = device()
    w = wl.TINY
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, 64), 64)


def test_kda_layer_config():
    """B=1 H=14 d=64 T=8192, per-key alpha, all heads checked."""
    dev = device()
    w = wl.KDA_LAYER
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, 64), 64)


def test_exact_integer_placement_bitwise():
    """alpha = beta = 1, one-hot keys k_t = e_{t mod d}, one-hot queries and
    small-integer values: every chunk product is exact in fp16 x fp16 -> fp32,
    so o, snapshots and final states equal the oracle bit for bit and every
    state column names the (sequence, position) that wrote it."""
    dev = device()
    import oracle
    d, H = 64, 2
    lens = [130, 0, 64, 1, 257, 4096 + 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    k = np.zeros((T, H, d), np.float32)
    q = np.zeros((T, H, d), np.float32)
    v = np.zeros((T, H, d), np.float32)
    for n, L in enumerate(lens):
        p = np.arange(L)
        t = cu[n] + p
        for h in range(H):
            k[t, h, (p + h) % d] = 1.0
            q[t, h, (5 * p + 3 * h) % d] = 1.0
            v[t, h, 0] = n + 1
            v[t, h, 1] = p % 128
            v[t, h, 2] = p // 128
            v[t, h, 3] = h
    to_bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)  # noqa: E731
    alpha = torch.ones((T, H, d), dtype=torch.float32, device=dev)
    beta = torch.ones((T, H), dtype=torch.float32, device=dev)
    interval = 64
    inp = dict(q=to_bf(q), k=to_bf(k), v=to_bf(v), alpha=alpha, beta=beta,
               cu_seqlens=torch.from_numpy(cu).to(dev), cu_seqlens_host=torch.from_numpy(cu),
               initial_state=None)
    o, fin, snaps = run_prefill(inp, interval)
    A = {n: wl.to_oracle_arrays(inp[n]) for n in ("q", "k", "v", "alpha", "beta")}
    o_r, f_r, s_r = oracle.run(A["q"], A["k"], A["v"], A["alpha"], A["beta"], cu, None, interval)
    assert snaps.shape[0] == s_r.shape[0] == sum(L // interval for L in lens)
    assert np.array_equal(o.cpu().numpy().astype(np.float64), o_r)
    assert np.array_equal(fin.cpu().numpy().astype(np.float64), f_r)
    assert np.array_equal(snaps.cpu().numpy().astype(np.float64), s_r)


def test_run_twice_bitwise_deterministic():
    dev = device()
    w = custom("determinism", H=4, d=128, lens=(500, 77, 1024), gate="per_key", interval=128, seed=13)
    inp = wl.make_prefill_inputs(w, dev)
    a = run_prefill(inp, w.interval)
    b = run_prefill(inp, w.interval)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d,gate", [(64, "per_key"), (128, "scalar")])
@pytest.mark.parametrize("segment_tokens", [0, 128])
def test_packed_equals_solo_bitwise(segment_tokens, d, gate):
    """With a fixed segment plan a sequence's results do not depend on the pack.
    A pack runs from the work table; a single sequence forms its work items in
    the kernels, so this also checks that both give the same items (at d = 128
    with the scalar gate, through the two-role map pass and output pass)."""
    dev = device()
    w = custom(f"packing_{d}_{gate}", H=2, d=d, lens=(300, 0, 65, 128, 700), gate=gate, interval=64, seed=14)
    inp = wl.make_prefill_inputs(w, dev)
    o, fin, snaps = run_prefill(inp, w.interval, segment_tokens)
    cu = inp["cu_seqlens_host"].tolist()
    slot = 0
    for n, L in enumerate(w.seq_lens):
        s, e = cu[n], cu[n + 1]
        sub = dict(q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e], alpha=inp["alpha"][s:e],
                   beta=inp["beta"][s:e], cu_seqlens=torch.tensor([0, L], device=dev),
                   cu_seqlens_host=torch.tensor([0, L]),
                   initial_state=inp["initial_state"][n:n + 1].contiguous())
        o1, f1, s1 = run_prefill(sub, w.interval, segment_tokens)
        assert torch.equal(o[s:e], o1)
        assert torch.equal(fin[n:n + 1], f1)
        assert torch.equal(snaps[slot:slot + s1.shape[0]], s1)
        slot += s1.shape[0]


def test_prefix_split_resume_bitwise():
    """Prefill of the first N tokens (N % 64 == 0), then the rest from its final
    state, equals the unsplit run bit for bit; the snapshot at N equals the
    prefix's final state."""
    dev = device()
    w = custom("prefix", H=2, d=128, lens=(1000,), gate="scalar", interval=256, seed=15)
    inp = wl.make_prefill_inputs(w, dev)
    o, fin, snaps = run_prefill(inp, w.interval, 0)
    N = 512
    part = lambda s, e, init: dict(q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e],  # noqa: E731
                                   alpha=inp["alpha"][s:e], beta=inp["beta"][s:e],
                                   cu_seqlens=torch.tensor([0, e - s], device=dev),
                                   cu_seqlens_host=torch.tensor([0, e - s]), initial_state=init)
    o1, f1, _ = run_prefill(part(0, N, inp["initial_state"]), 0, 0)
    o2, f2, _ = run_prefill(part(N, 1000, f1), 0, 0)
    assert torch.equal(snaps[1], f1[0])
    assert torch.equal(o[:N], o1) and torch.equal(o[N:], o2) and torch.equal(fin, f2)


@pytest.mark.parametrize("segment_tokens", [64, 128, 192, 1024])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
def test_segmented_plan_matches_oracle(segment_tokens, gate):
    """Forced segment plans (segment maps, fp32 scan, reruns) on a varlen pack
    with snapshots and initial states. At d=128 with the scalar gate and bf16
    inputs the reruns are the two-role pass-3 kernel: segments of one chunk
    (nothing to prepare ahead), two chunks (no chunk after the next) and more,
    with ragged last segments."""
    dev = device()
    w = custom(f"seg_{segment_tokens}_{gate}", H=2, d=128, lens=(2000, 70, 0, 1280, 64), gate=gate,
               interval=128, seed=16)
    print(f"case {w.name} lens={w.seq_lens}", flush=True)
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, w.interval, segment_tokens), w.interval)


def test_segmented_close_to_unsegmented():
    dev = device()
    w = custom("seg_vs_plain", H=3, d=64, lens=(5000,), gate="per_key", interval=0, seed=17)
    inp = wl.make_prefill_inputs(w, dev)
    a = run_prefill(inp, 0, 0)
    b = run_prefill(inp, 0, 512)
    for x, y in zip(a[:2], b[:2]):
        assert (x - y).abs().max().item() <= 1e-3 * x.abs().max().item()


def test_long_prefill_config_all_heads():
    """B=1 H=16 d=128 T=262144, scalar alpha, the measured launch (automatic
    segment plan); the oracle checks all 16 heads over the whole sequence."""
    dev = device()
    w = wl.LONG_PREFILL
    inp = wl.make_prefill_inputs(w, dev)
    outs = run_prefill(inp, 0)
    check_prefill(inp, outs, 0)


@pytest.mark.parametrize("group", range(4))
def test_varlen_config_all_heads(group):
    """32 packed sequences, H=32 d=128, per-key alpha, initial states,
    snapshots every 4096 tokens; the oracle checks every sequence, snapshot
    and final state of 8 of the 32 heads per case (all heads over the four
    cases; each case runs the full launch)."""
    dev = device()
    w = wl.VARLEN
    inp = wl.make_prefill_inputs(w, dev)
    outs = run_prefill(inp, w.interval)
    assert outs[2].shape[0] == sum(L // w.interval for L in w.seq_lens)
    print(f"varlen heads {8 * group}..{8 * group + 7}", flush=True)
    check_prefill(inp, outs, w.interval, heads=range(8 * group, 8 * group + 8))


@pytest.mark.parametrize("segment_tokens", [0, 64, -1])
def test_initial_state_may_alias_final_state(segment_tokens):
    """final_state may be the initial_state buffer: results equal those of a
    run with separate buffers, bit for bit, also when a split sequence's
    segments (more workgroups than compute units at 64-token segments) run
    in one pass."""
    dev = device()
    w = custom(f"alias_{segment_tokens}", H=8, d=64, lens=(4096, 300, 0, 1000), gate="per_key", seed=18)
    inp = wl.make_prefill_inputs(w, dev)
    o_ref, f_ref, _ = run_prefill(inp, 0, segment_tokens)
    state = inp["initial_state"].clone()
    o = torch.empty_like(o_ref)
    snaps = torch.empty((0,) + tuple(f_ref.shape[1:]), dtype=torch.float32, device=dev)
    kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["cu_seqlens"], state, 0,
                        cu_seqlens_host=inp["cu_seqlens_host"], segment_tokens=segment_tokens,
                        out=(o, state, snaps))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(state, f_ref)


def test_snapshots_to_pinned_host_memory_bitwise():
    """Snapshots written straight into pinned host memory by the kernels equal
    the device-memory snapshots bit for bit (segmented and plain plans)."""
    dev = device()
    w = custom("host_snaps", H=4, d=128, lens=(3000, 64, 0, 1300), gate="per_key", interval=128, seed=19)
    inp = wl.make_prefill_inputs(w, dev)
    for seg in (0, -1):
        o_d, f_d, s_d = run_prefill(inp, w.interval, seg)
        o_h, f_h, s_h = kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                            inp["cu_seqlens"], inp["initial_state"], w.interval,
                                            cu_seqlens_host=inp["cu_seqlens_host"], segment_tokens=seg,
                                            snapshots_on_host=True)
        torch.cuda.synchronize()
        assert s_h.device.type == "cpu" and s_h.is_pinned()
        assert torch.equal(s_h, s_d.cpu()) and torch.equal(o_h, o_d) and torch.equal(f_h, f_d)
        # and the host snapshots (with o and the final states of that call)
        # against the oracle
        check_prefill(inp, (o_h, f_h, s_h), w.interval)


def test_pageable_host_snapshots_rejected_by_binding():
    dev = device()
    w = custom("pageable", H=1, d=64, lens=(128,), gate="scalar", interval=64, seed=20)
    inp = wl.make_prefill_inputs(w, dev)
    o = torch.empty((128, 1, 64), dtype=torch.float32, device=dev)
    fin = torch.empty((1, 1, 64, 64), dtype=torch.float32, device=dev)
    snaps = torch.empty((2, 1, 64, 64), dtype=torch.float32)          # pageable
    with pytest.raises(ValueError):
        kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["cu_seqlens"],
                            inp["initial_state"], w.interval, cu_seqlens_host=inp["cu_seqlens_host"],
                            out=(o, fin, snaps))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
def test_segmented_every_variant(d, dtype, gate):
    """Forced 128-token segments for every (d, input dtype, gate) variant: the
    map pass, its stored W and U', the scan, the output pass of the split
    sequences and that of the whole ones, on a varlen pack with a ragged tail,
    snapshots and initial states."""
    dev = device()
    w = custom(f"segvar_{d}_{dtype}_{gate}", H=2, d=d, lens=(700, 130, 0, 64), gate=gate, dtype=dtype,
               interval=64, seed=21)
    print(f"case {w.name}", flush=True)
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, w.interval, 128), w.interval)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("segment_tokens", [0, 128])
def test_rectangular_heads(dk, dv, gate, dtype, segment_tokens):
    """d_k != d_v: the state is d_v x d_k. d_v = 2 d_k runs every head as two
    value heads of d_k rows that share q, k and the gates; d_k = 2 d_v pads
    the values and states with zero rows. Varlen pack with a ragged tail,
    snapshots and initial states, plain and segmented plans."""
    dev = device()
    w = custom(f"rect_{dk}x{dv}_{gate}_{dtype}_{segment_tokens}", H=3, d=dk, dv=dv, lens=(700, 130, 0, 64, 1),
               gate=gate, dtype=dtype, interval=64, seed=22)
    print(f"case {w.name}", flush=True)
    inp = wl.make_prefill_inputs(w, dev)
    check_prefill(inp, run_prefill(inp, w.interval, segment_tokens), w.interval)


def test_rectangular_heads_alias_and_host_snapshots():
    """d_k = 2 d_v through the padded path: the final state written over the
    initial state, and the snapshots into pinned host memory, against the
    oracle."""
    dev = device()
    w = custom("rect_alias", H=2, d=128, dv=64, lens=(500, 129), gate="per_key", interval=128, seed=23)
    inp = wl.make_prefill_inputs(w, dev)
    init0 = inp["initial_state"].clone()
    state = inp["initial_state"].clone()
    n_snap = kda.kda_snapshot_count(inp["cu_seqlens_host"], w.interval)
    o = torch.empty((w.T, w.H, w.dv), dtype=torch.float32, device=dev)
    snaps = torch.empty((n_snap, w.H, w.dv, w.dk), dtype=torch.float32, pin_memory=True)
    kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["cu_seqlens"], state,
                        w.interval, cu_seqlens_host=inp["cu_seqlens_host"], out=(o, state, snaps))
    torch.cuda.synchronize()
    inp["initial_state"] = init0
    check_prefill(inp, (o, state, snaps), w.interval)


def _near_limit_alpha(inp, exponent, block):
    """Per-key alpha whose product over every aligned block of `block` tokens
    is 2^-exponent in key channels 0..7 of every head (the others keep their
    sigmoid draws): the narrowest decay the chunked kernels accept."""
    a = inp["alpha"].clone()
    a[:, :, :8] = 2.0 ** (-exponent / block)
    return a


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("segment_tokens", [0, 128])
def test_per_key_decay_at_the_forward_limit(d, segment_tokens):
    """Key channels whose decay over each aligned 16-token block is 2^-99.5,
    just inside the prefill's stated limit of 2^-100 (the per-key Gram
    products are taken relative to each block's first token): o, snapshots
    and final states still within tolerance of the oracle."""
    dev = device()
    w = custom(f"pk_limit_{d}_{segment_tokens}", H=2, d=d, lens=(300, 64 + 17, 0, 16), gate="per_key",
               interval=64, seed=24)
    inp = wl.make_prefill_inputs(w, dev)
    inp["alpha"] = _near_limit_alpha(inp, 99.5, 16)
    check_prefill(inp, run_prefill(inp, w.interval, segment_tokens), w.interval)


@pytest.mark.parametrize("n_seqs,hi,d,gate", [(3000, 300, 64, "per_key"), (2000, 200, 128, "scalar"),
                                              (9000, 40, 64, "per_key")])
def test_many_short_sequences(n_seqs, hi, d, gate):
    """Thousands of short packed sequences (lengths U[0, hi], empty ones
    included) with snapshots every 64 tokens: up to 8192 sequences the work
    table is sorted longest first, beyond that it keeps sequence order; every
    sequence, snapshot and final state against the oracle."""
    rng = np.random.Generator(np.random.PCG64(90 + d))
    lens = tuple(int(x) for x in rng.integers(0, hi, endpoint=True, size=n_seqs))
    w = custom(f"many_{n_seqs}_{d}_{gate}", H=2 if n_seqs < 8192 else 1, d=d, lens=lens, gate=gate,
               interval=64, seed=91)
    inp = wl.make_prefill_inputs(w, device())
    outs = run_prefill(inp, w.interval)
    assert outs[2].shape[0] == sum(L // 64 for L in lens)
    check_prefill(inp, outs, w.interval)
