"""GPU parity of kda_decode_step against the fp64 CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_72_amd as kda
import oracle
from gated_delta_rule_72_amd import workloads as wl

from gpu_util import O_TOL, STATE_TOL, device

pytestmark = pytest.mark.gpu


def _check_decode(di, s0, o, heads=None):
    B, H = di["q"].shape[:2]
    hs = list(range(H)) if heads is None else list(heads)
    idx = torch.tensor(hs, device=di["q"].device)
    sel = lambda t: t.index_select(1, idx)  # noqa: E731
    A = {n: wl.to_oracle_arrays(sel(di[n])) for n in ("q", "k", "v", "alpha", "beta")}
    cu = np.arange(B + 1, dtype=np.int64)   # B sequences of one token each
    rc, rep = oracle.ref_check(A["q"], A["k"], A["v"], A["alpha"], A["beta"], cu,
                               sel(s0).cpu().numpy(), 0, sel(o).cpu().numpy(),
                               sel(di["state"]).cpu().numpy(), None, O_TOL, STATE_TOL)
    print(f"oracle report: {rep}", flush=True)
    assert rc == oracle.OK, rep


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_small(d, gate, dtype):
    dev = device()
    w = wl.DECODE.with_(dk=d, dv=d, H=3, seq_lens=(1,) * 5, gate=gate, dtype=dtype, seed=21)
    di = wl.make_decode_inputs(w, dev)
    s0 = di["state"].clone()
    o = kda.decode_step(di["q"], di["k"], di["v"], di["alpha"], di["beta"], di["state"])
    torch.cuda.synchronize()
    _check_decode(di, s0, o)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
@pytest.mark.parametrize("gate", ["scalar", "per_key"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_rectangular_heads(dk, dv, gate, dtype):
    """d_k != d_v: d_v/32 wavefronts of 32 state rows, rows d_k/4 lanes wide."""
    dev = device()
    w = wl.DECODE.with_(dk=dk, dv=dv, H=3, seq_lens=(1,) * 5, gate=gate, dtype=dtype, seed=23)
    di = wl.make_decode_inputs(w, dev)
    s0 = di["state"].clone()
    o = kda.decode_step(di["q"], di["k"], di["v"], di["alpha"], di["beta"], di["state"])
    torch.cuda.synchronize()
    _check_decode(di, s0, o)


def test_decode_config_full():
    """B=256 H=16 d=128 per-key alpha; every (sequence, head) checked."""
    dev = device()
    di = wl.make_decode_inputs(wl.DECODE, dev)
    s0 = di["state"].clone()
    o = kda.decode_step(di["q"], di["k"], di["v"], di["alpha"], di["beta"], di["state"])
    torch.cuda.synchronize()
    _check_decode(di, s0, o)


def test_decode_equals_one_token_prefill():
    dev = device()
    w = wl.DECODE.with_(H=4, seq_lens=(1,) * 6, seed=22)
    di = wl.make_decode_inputs(w, dev)
    s0 = di["state"].clone()
    o_dec = kda.decode_step(di["q"], di["k"], di["v"], di["alpha"], di["beta"], di["state"])
    B = w.num_seqs
    cu = torch.arange(B + 1, dtype=torch.int64)
    o_pre, fin, _ = kda.prefill_chunked(di["q"], di["k"], di["v"], di["alpha"], di["beta"],
                                        cu.to(dev), s0, 0, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    # both paths are each within 2e-3 / 1e-3 of the oracle; the prefill's
    # products run on fp16 MFMA, the decode step in fp32
    scale_o = o_pre.abs().max().item()
    scale_s = fin.abs().max().item()
    assert (o_dec - o_pre).abs().max().item() <= 2e-3 * scale_o
    assert (di["state"] - fin).abs().max().item() <= 1e-3 * scale_s


def test_chained_decode_matches_prefill():
    """T decode steps over one sequence agree with one chunked prefill."""
    dev = device()
    T, H, d = 150, 2, 64
    w = wl.Workload("chain", H=H, dk=d, dv=d, seq_lens=(T,), gate="per_key", s0_std=0.02, seed=23)
    inp = wl.make_prefill_inputs(w, dev)
    o_pre, fin, _ = kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                        inp["cu_seqlens"], inp["initial_state"], 0)
    state = inp["initial_state"].clone()            # [1, H, d, d]
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(inp["q"][t:t + 1], inp["k"][t:t + 1], inp["v"][t:t + 1],
                                    inp["alpha"][t:t + 1], inp["beta"][t:t + 1], state))
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, 0)
    assert (o_dec - o_pre).abs().max().item() <= 2e-3 * o_pre.abs().max().item()
    assert (state - fin).abs().max().item() <= 1e-3 * fin.abs().max().item()
