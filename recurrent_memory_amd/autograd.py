"""torch.autograd binding of the chunkwise forward and backward.

``delta_rule(variant, q, k, v, beta, g=None, wgate=None, S0=None)`` returns
(o, S_T) like ``ops.delta_fwd`` and differentiates through ``ops.delta_bwd``:
the forward and the backward both run in the library's kernels, this module
only routes tensors.  Gradients flow to every tensor argument that requires
them (grouped query/key heads included); the backward recomputes the forward
states itself, so nothing but the inputs is saved.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import ops


class _DeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, variant, q, k, v, beta, g, wgate, S0):
        o, S_T = ops.delta_fwd(variant, q, k, v, beta, wgate=wgate, g=g, S0=S0)
        ctx.variant = variant
        ctx.save_for_backward(q, k, v, beta, g, wgate, S0)
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, beta, g, wgate, S0 = ctx.saved_tensors
        if dO is None:
            dO = torch.zeros(v.shape, dtype=v.dtype, device=v.device)
        dO = dO.contiguous().to(v.dtype)
        if dS_T is not None:
            dS_T = dS_T.contiguous().to(torch.float32)
        gr = ops.delta_bwd(ctx.variant, q, k, v, beta, dO, g=g, S0=S0, dS_T=dS_T, wgate=wgate,
                           want_dS0=S0 is not None and ctx.needs_input_grad[7])
        return (None, gr["dq"], gr["dk"], gr["dv"], gr["dbeta"], gr["dg"], gr["dwgate"], gr["dS0"])


def delta_rule(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               beta: torch.Tensor, g: Optional[torch.Tensor] = None,
               wgate: Optional[torch.Tensor] = None, S0: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable chunkwise forward: (o, S_T) with gradients through delta_bwd."""
    return _DeltaRule.apply(variant, q, k, v, beta, g, wgate, S0)
