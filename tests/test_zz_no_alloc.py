"""The allocation-free prefill (kda_prefill_chunked_noalloc, through the C ABI)
against kda_prefill_chunked with segment_tokens = 0: the same kernels on the
same plan, so o, final states and snapshots must agree bit for bit. Two calls
in a row share the library's static scratch; the second is smaller, so a work
table left over from the first must not leak into it."""
import pytest
import torch

import gated_delta_rule_72_amd as kda
from gated_delta_rule_72_amd import workloads as wl

from gpu_util import check_prefill, custom, device

pytestmark = pytest.mark.gpu


def _noalloc(inp, w):
    dev = inp["q"].device
    T, H = w.T, w.H
    n_snap = kda.kda_snapshot_count(inp["cu_seqlens_host"], w.interval)
    o = torch.empty((T, H, w.dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.num_seqs, H, w.dv, w.dk), dtype=torch.float32, device=dev)
    snaps = torch.empty((n_snap, H, w.dv, w.dk), dtype=torch.float32, device=dev)
    shape = kda.make_shape(H, w.dk, w.dv, inp["q"].dtype, w.gate == "per_key")
    kda.kda_prefill_chunked_noalloc(shape, inp["cu_seqlens_host"], inp["cu_seqlens"], inp["q"], inp["k"], inp["v"],
                                    inp["alpha"], inp["beta"], inp["initial_state"], o, fin,
                                    snaps if n_snap else None, snapshot_interval=w.interval)
    torch.cuda.synchronize()
    return o, fin, snaps


@pytest.mark.parametrize("d,gate", [(64, "per_key"), (128, "scalar")])
def test_noalloc_prefill_matches_workspace_entry_point(d, gate):
    dev = device()
    big = custom(f"noalloc_big_{d}", H=4, d=d, lens=(900, 3, 0, 260, 64, 1200, 17), gate=gate, interval=64, seed=41)
    small = custom(f"noalloc_small_{d}", H=2, d=d, lens=(70, 130), gate=gate, interval=64, seed=42)
    for w in (big, small):
        print(f"case {w.name} lens={w.seq_lens}", flush=True)
        inp = wl.make_prefill_inputs(w, dev)
        got = _noalloc(inp, w)
        ref = kda.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["cu_seqlens"],
                                  inp["initial_state"], w.interval, cu_seqlens_host=inp["cu_seqlens_host"],
                                  segment_tokens=0)
        torch.cuda.synchronize()
        for x, r in zip(got, ref):
            assert torch.equal(x, r)
        check_prefill(inp, got, w.interval)
