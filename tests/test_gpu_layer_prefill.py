"""GPU parity of kda_layer_prefill (the recurrence and the KDA layer back end
in one call) through the C ABI.

Against kda_prefill_chunked followed by kda_layer_back with the gate logits
widened to fp32: bit for bit, in the fused forms (bf16 inputs with the scalar
gate at d = 128 or the per-key gate at d = 64, every sequence split: the back
end runs on each chunk's output tile on chip and forms the row sums of
squares in the back-end kernel's order) and in the composed one (every other
shape and plan). Against the fp64 oracle (token
recurrence of oracle/kda_oracle.c, back end of oracle/layer.py): max error over
a (sequence, head) slice relative to that slice's max |reference|, 5e-3 for
bf16 out (the recurrence's 2e-3, which RMSNorm rescales per token, and one
bf16 rounding, 2^-9).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_72_amd as kda
from gated_delta_rule_72_amd import workloads as wl
from oracle import layer as L

from gpu_util import custom, device

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    dev = device()
    inp = wl.make_prefill_inputs(w, dev)
    li = wl.make_layer_inputs(w, dev, seed=seed)
    g = li["g_logit"].to(inp["q"].dtype)
    return inp, g, li["norm_w"]


def _separate(inp, g, norm_w, interval, seg, out_dtype):
    o, fin, snaps = kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["cu_seqlens"],
                                        inp["initial_state"], interval, cu_seqlens_host=inp["cu_seqlens_host"],
                                        segment_tokens=seg)
    y = kda.layer_back(o, g.float(), norm_w, 1e-6, out_dtype)
    return y, fin, snaps


def _fused(inp, g, norm_w, interval, seg, out_dtype):
    return kda.layer_prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], g, norm_w, 1e-6,
                             inp["cu_seqlens"], inp["initial_state"], interval,
                             cu_seqlens_host=inp["cu_seqlens_host"], segment_tokens=seg, out_dtype=out_dtype)


def _fused_form(w, seg):
    """Whether kda_layer_prefill takes the fused form for this workload."""
    if w.dtype != "bf16" or w.dk != w.dv or (w.dk, w.gate) not in ((128, "scalar"), (64, "per_key")):
        return False
    if seg == 0:
        return False
    if seg < 0:
        if w.num_seqs * w.H >= torch.cuda.get_device_properties(0).multi_processor_count:
            return False
        total = sum((n + 63) // 64 for n in w.seq_lens) * w.H
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        seg = max((total + cus - 1) // cus, 8) * 64
    return all(n == 0 or n > seg for n in w.seq_lens)


CASES = [
    # fused: every non-empty sequence longer than the segment, ragged tails, an empty one
    ("fused_pack", dict(H=2, d=128, lens=(1100, 0, 641, 300), dtype="bf16", gate="scalar"), 256, 128, True),
    # fused, automatic plan on one sequence
    ("fused_auto", dict(H=2, d=128, lens=(4096 + 33,), dtype="bf16", gate="scalar"), -1, 0, True),
    # fused, the KDA layer's form (per-key gate, d = 64)
    ("fused_pk64", dict(H=2, d=64, lens=(1100, 0, 641, 300), dtype="bf16", gate="per_key"), 256, 128, True),
    # composed: a sequence stays whole
    ("mixed", dict(H=2, d=128, lens=(1100, 100), dtype="bf16", gate="scalar"), 256, 0, False),
    # composed: unsegmented plans, per-key gate at d = 128, fp32 inputs
    ("unsegmented", dict(H=3, d=128, lens=(700, 65), dtype="bf16", gate="scalar"), 0, 64, False),
    ("per_key_d128", dict(H=2, d=128, lens=(700, 300), dtype="bf16", gate="per_key"), 256, 0, False),
    ("per_key_d64", dict(H=2, d=64, lens=(150, 7, 64), dtype="bf16", gate="per_key"), -1, 64, False),
    ("fp32_d64", dict(H=2, d=64, lens=(300,), dtype="fp32"), 128, 0, False),
]


@pytest.mark.parametrize("name,kw,seg,interval,fused", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_layer_prefill_matches_separate_calls(name, kw, seg, interval, fused, out_dtype):
    w = custom(f"lp_{name}", s0_std=0.02, seed=61, **kw)
    assert _fused_form(w, seg) == fused
    inp, g, norm_w = _inputs(w, 62)
    y, fin, snaps = _fused(inp, g, norm_w, interval, seg, out_dtype)
    y_ref, fin_ref, snaps_ref = _separate(inp, g, norm_w, interval, seg, out_dtype)
    torch.cuda.synchronize()
    print(f"{name}: fused form {fused}, out {tuple(y.shape)} {y.dtype}", flush=True)
    assert y.dtype == out_dtype
    if not torch.equal(y, y_ref):
        d = (y.float() - y_ref.float()).abs()
        idx = torch.nonzero(d).tolist()[:4]
        raise AssertionError(f"{int((d > 0).sum())} elements differ, max {float(d.max()):.3e}, first {idx}")
    assert torch.equal(fin, fin_ref)
    assert torch.equal(snaps, snaps_ref)


def _oracle_out(inp, g, norm_w, heads=None, threads=16):
    import oracle
    cu = inp["cu_seqlens_host"].numpy()
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    arr = lambda t: sel(wl.to_oracle_arrays(t))  # noqa: E731
    s0 = inp["initial_state"]
    s0 = None if s0 is None else (s0.cpu().numpy() if heads is None else s0[:, heads].cpu().numpy())
    ro, _, _ = oracle.run(arr(inp["q"]), arr(inp["k"]), arr(inp["v"]), arr(inp["alpha"]), arr(inp["beta"]), cu, s0, 0,
                          threads=threads)
    return L.layer_back(ro, arr(g), wl.to_oracle_arrays(norm_w), 1e-6)


def _rel_slices(y, ref, cu):
    worst = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(ref.shape[1]):
            r = ref[s:e, h]
            if r.size:
                worst = max(worst, float(np.max(np.abs(y[s:e, h] - r)) / max(np.max(np.abs(r)), 1e-30)))
    return worst


@pytest.mark.parametrize("name,kw,seg", [("fused_pack", CASES[0][1], 256), ("fused_pk64", CASES[2][1], 256),
                                         ("per_key_d64", dict(H=2, d=64, lens=(150, 7, 64), dtype="bf16",
                                                              gate="per_key"), -1)],
                         ids=["fused", "fused_pk64", "composed"])
def test_layer_prefill_matches_oracle(name, kw, seg):
    w = custom(f"lp_{name}", s0_std=0.02, seed=61, **kw)
    inp, g, norm_w = _inputs(w, 62)
    y, _, _ = _fused(inp, g, norm_w, 0, seg, torch.bfloat16)
    torch.cuda.synchronize()
    ref = _oracle_out(inp, g, norm_w)
    err = _rel_slices(y.float().cpu().numpy().astype(np.float64), ref, inp["cu_seqlens_host"].numpy())
    print(f"{name}: out vs oracle {err:.3e}", flush=True)
    assert err <= 5e-3


def test_layer_prefill_long_prefill_shape():
    """The long-prefill workload (T = 262144, H = 16, d = 128, scalar gate,
    bf16) in the launch configuration the benchmark times (automatic plan, the
    fused form): out equal bit for bit to the separate calls on every head,
    and against the oracle on heads 0 and 15."""
    w = wl.LONG_PREFILL
    assert _fused_form(w, -1)
    inp, g, norm_w = _inputs(w, 63)
    y, fin, _ = _fused(inp, g, norm_w, 0, -1, torch.bfloat16)
    y_ref, fin_ref, _ = _separate(inp, g, norm_w, 0, -1, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(fin, fin_ref)
    del y_ref, fin_ref
    heads = [0, 15]
    ref = _oracle_out(inp, g, norm_w, heads)
    err = _rel_slices(y[:, heads].float().cpu().numpy().astype(np.float64), ref, inp["cu_seqlens_host"].numpy())
    print(f"long prefill: out vs oracle (heads {heads}) {err:.3e}", flush=True)
    assert err <= 5e-3


def test_layer_prefill_kda_layer_shape():
    """The KDA-layer workload (T = 8192, H = 14, d = 64, per-key gate, bf16)
    with the automatic plan (the fused form): out equal bit for bit to the
    separate calls and within tolerance of the oracle, every head."""
    w = wl.KDA_LAYER
    assert _fused_form(w, -1)
    inp, g, norm_w = _inputs(w, 64)
    y, fin, _ = _fused(inp, g, norm_w, 0, -1, torch.bfloat16)
    y_ref, fin_ref, _ = _separate(inp, g, norm_w, 0, -1, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(fin, fin_ref)
    ref = _oracle_out(inp, g, norm_w)
    err = _rel_slices(y.float().cpu().numpy().astype(np.float64), ref, inp["cu_seqlens_host"].numpy())
    print(f"KDA layer shape: out vs oracle {err:.3e}", flush=True)
    assert err <= 5e-3
