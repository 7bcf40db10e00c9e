"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import gated_delta_rule_72_amd as kda
import oracle
from gated_delta_rule_72_amd import workloads as wl

O_TOL = 2e-3       # max relative error on o (slice-max normalised)
STATE_TOL = 1e-3   # on final states and snapshots


def device():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_prefill(inp: dict, interval: int, segment_tokens: int = -1):
    o, fin, snaps = kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                        inp["cu_seqlens"], inp["initial_state"], interval,
                                        cu_seqlens_host=inp["cu_seqlens_host"],
                                        segment_tokens=segment_tokens)
    torch.cuda.synchronize()
    return o, fin, snaps


def check_prefill(inp: dict, outs, interval: int, heads=None, o_tol=O_TOL, state_tol=STATE_TOL,
                  threads: int = 0):
    """Compares GPU outputs with the oracle on the selected heads (all by
    default). Returns the oracle's report; asserts the tolerances."""
    o, fin, snaps = outs
    H = inp["q"].shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    sel = lambda t, ax: None if t is None else t.index_select(ax, torch.tensor(hs, device=t.device))  # noqa: E731
    A = {n: wl.to_oracle_arrays(sel(inp[n], 1)) for n in ("q", "k", "v", "alpha", "beta")}
    init = inp["initial_state"]
    init = None if init is None else sel(init, 1).cpu().numpy()
    rc, rep = oracle.ref_check(A["q"], A["k"], A["v"], A["alpha"], A["beta"],
                               inp["cu_seqlens_host"].numpy(), init, interval,
                               sel(o, 1).cpu().numpy(), sel(fin, 1).cpu().numpy(),
                               sel(snaps, 1).cpu().numpy() if snaps is not None and snaps.numel() else None,
                               o_tol, state_tol, threads)
    print(f"oracle report: {rep}", flush=True)
    assert rc == oracle.OK, rep
    return rep


def custom(name, H, d, lens, gate="per_key", dtype="bf16", s0_std=0.02, interval=0, seed=0,
           alpha_bias=5.0, alpha_std=1.0, dv=None):
    return wl.Workload(name, H=H, dk=d, dv=d if dv is None else dv, seq_lens=tuple(lens), dtype=dtype, gate=gate,
                       alpha_bias=alpha_bias, alpha_std=alpha_std, s0_std=s0_std, interval=interval,
                       seed=seed)
