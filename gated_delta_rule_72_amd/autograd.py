"""torch.autograd glue: the chunked prefill as a differentiable function.

Forward is kda_prefill_chunked, backward is kda_prefill_backward (which
recomputes the forward's states inside); this module only routes tensors and
gradients between them and torch's autograd. Gradients of q, k, v come back
in the dtype of the inputs (the library computes them in fp32).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import kda


class _ChunkedGatedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host):
        o, final, _ = kda.prefill_chunked(q, k, v, alpha, beta, cu_seqlens, initial_state, 0,
                                          cu_seqlens_host=cu_seqlens_host)
        ctx.save_for_backward(q, k, v, alpha, beta, initial_state, cu_seqlens)
        ctx.cu_seqlens_host = cu_seqlens_host
        return o, final

    @staticmethod
    def backward(ctx, d_o, d_final):
        q, k, v, alpha, beta, initial_state, cu_seqlens = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros((q.shape[0], q.shape[1], v.shape[2]), dtype=torch.float32, device=q.device)
        want_init = initial_state is not None and ctx.needs_input_grad[5]
        dq, dk, dv, dalpha, dbeta, d_init = kda.prefill_backward(
            q, k, v, alpha, beta, d_o.float().contiguous(), cu_seqlens, initial_state,
            None if d_final is None else d_final.float().contiguous(), cu_seqlens_host=ctx.cu_seqlens_host,
            want_d_initial=want_init)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dalpha, dbeta,
                d_init if want_init else None, None, None)


def gated_delta_rule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                     cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                     cu_seqlens_host: Optional[torch.Tensor] = None):
    """Differentiable chunked prefill: returns (o [T,H,dv] fp32, final_state
    [N,H,dv,dk] fp32). Shapes and dtypes as kda.prefill_chunked."""
    T = q.shape[0]
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int64, device=q.device)
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.to("cpu")
    return _ChunkedGatedDeltaRule.apply(q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host)
