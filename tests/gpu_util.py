"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path through
the C ABI, and measure errors against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import CHANNEL_LOG_DECAY_FLOOR

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
# max relative error per [batch, head] slice (max |x - ref| / max |ref|)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(x, dtype="f32"):
    """Upload a float32 numpy array (already representable in ``dtype``) exactly."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(TORCH_DTYPE[dtype])
    return t.cuda()


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def gpu_fwd(variant, x, dtype, want_state=True, in_place=False):
    S0 = dev(x["S0"], "f32") if x.get("S0") is not None else None
    kw = {}
    if in_place:
        if S0 is None:
            raise ValueError("in-place needs S0")
        kw["S_T"] = S0
    o, ST = ops.delta_fwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype),
                          dev(x["beta"], dtype), wgate=dev(x.get("wgate"), dtype),
                          g=dev(x.get("g"), dtype), S0=S0, want_state=want_state, **kw)
    torch.cuda.synchronize()
    return host(o), host(ST)


def slice_rel_err(x, ref, head_axes):
    """max over (batch, head) slices of max|x-ref| / max|ref|.  head_axes: the axes
    that index (batch, head); all others are reduced inside the slice."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    axes = tuple(a for a in range(x.ndim) if a not in head_axes)
    num = np.abs(x - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def errs(o, S, o_ref, S_ref):
    """(o error, S error) per the slice metric; o is [B,T,H,dv], S is [B,H,dv,dk]."""
    eo = slice_rel_err(o, o_ref, (0, 2))
    es = slice_rel_err(S, S_ref, (0, 1)) if S is not None and S_ref is not None else 0.0
    return eo, es


def announce(*parts):
    """Name the case on the real stderr (past pytest's capture) before a GPU step."""
    import sys
    sys.__stderr__.write("[gpu case] " + " ".join(str(p) for p in parts) + "\n")
    sys.__stderr__.flush()


LOG_DECAY_FLOOR = float(CHANNEL_LOG_DECAY_FLOOR)   # per-token floor of channel log-decays (include/deltarule.h)


def floor_gates(shape, dtype, seed):
    """Channel log-decays in [-4, 0] with a share at -10 per token, below the
    floor: every channel of tokens 20..39 and channel 3 of every token."""
    from recurrent_memory_amd.inputs import round_to_bf16
    rng = np.random.default_rng(seed)
    g = (-rng.uniform(0, 4, shape)).astype(np.float32)
    g[:, 20:40] = -10.0
    g[..., 3] = -10.0
    return g if dtype == "f32" else round_to_bf16(g)
