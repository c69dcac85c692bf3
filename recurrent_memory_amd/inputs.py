"""Seeded synthetic workloads for the gated delta-rule forward and decode paths.

This module only draws random numbers and shapes them into the tensors a
recurrent-memory layer would hand to its mixing operator: L2-normalised
queries and keys, values, step sizes in (0, 1), log-decays <= 0 and an
initial state.  It contains none of the recurrence's arithmetic, so both the
HIP path and the CPU oracle can consume what it produces without sharing any
of the method.

Recipe (one generator per workload, ``numpy.random.PCG64(seed)``):

* draw order: q, k, v, then the step-size logits (for the split-gate form:
  erase logits, then write logits), then the decay logits, then S0;
* every draw is float32 ``standard_normal``;
* q and k are divided by their L2 norm per (batch, token, head) in float32;
* step sizes (per key channel for fg2) and split gates are ``sigmoid(z)``;
  log-decays are ``-softplus(z)`` (so the per-token decay ``exp(g)`` lies in
  (0, 1));
* S0 is ``0.02 * z`` where the workload asks for a random initial state;
* grouped value heads (``qk_heads`` < H): q and k are drawn with ``qk_heads``
  heads instead of H, in the same draw order;
* ``key_norm`` scales the normalised keys (1 by default; larger values give
  the high-energy keys of the exact-flow step-size tests);
* everything is then rounded to the workload dtype (round-to-nearest-even
  for bfloat16).  The rounded arrays are *the* inputs for every consumer.

The head width (d = 64 or 128), 16 heads and sequence lengths up to 32K follow
the memory-layer shapes of the DeltaTTT summary (paperlayer.ai, App. C: 16
memory heads; §5.4/Table 4: 32K training length).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

VARIANTS = ("deltanet", "gdn", "kda", "gdn2", "fg2")
DTYPES = ("f32", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str
    dtype: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int = 64
    random_s0: bool = False
    seed: int = 0


# The five synthetic workloads: four chunkwise forwards and one decode step.
WORKLOADS: Dict[str, Workload] = {
    "deltanet_fp32_t256_d64": Workload("deltanet_fp32_t256_d64", "deltanet", "f32",
                                       B=1, H=1, T=256, dk=64, dv=64, seed=1001),
    "gdn_bf16_b4_h16_t4096_d128": Workload("gdn_bf16_b4_h16_t4096_d128", "gdn", "bf16",
                                           B=4, H=16, T=4096, dk=128, dv=128, seed=1002),
    "kda_bf16_b2_h16_t8192_d128": Workload("kda_bf16_b2_h16_t8192_d128", "kda", "bf16",
                                           B=2, H=16, T=8192, dk=128, dv=128,
                                           random_s0=True, seed=1003),
    "gdn2_bf16_b1_h16_t32768_d128": Workload("gdn2_bf16_b1_h16_t32768_d128", "gdn2", "bf16",
                                             B=1, H=16, T=32768, dk=128, dv=128,
                                             random_s0=True, seed=1004),
    # single-token decode: T is 1 per step, the state is random
    "gdn_decode_bf16_b256_h16_d128": Workload("gdn_decode_bf16_b256_h16_d128", "gdn", "bf16",
                                              B=256, H=16, T=1, dk=128, dv=128,
                                              random_s0=True, seed=1005),
}

PREFILL_HEADLINE = "gdn_bf16_b4_h16_t4096_d128"
DECODE_HEADLINE = "gdn_decode_bf16_b256_h16_d128"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Finite inputs only (the generators never produce inf or NaN).
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _unit(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z, dtype=np.float32))).astype(np.float32)


def _neg_softplus(z: np.ndarray) -> np.ndarray:
    return (-np.logaddexp(np.float32(0.0), z)).astype(np.float32)


# Channel log-decays are drawn at or above -85/16, the per-token floor that the
# library applies when it loads a channel gate (include/deltarule.h), so both
# sides of a comparison see the same gates.  At gate_scale 1 a draw falls below
# it with probability about 5e-8 per entry; tests of the floor itself set gates
# below it explicitly.
CHANNEL_LOG_DECAY_FLOOR = np.float32(-85.0 / 16.0)


def draw(rng: np.random.Generator, variant: str, dtype: str, lead: tuple, dk: int, dv: int,
         gate_scale: float = 1.0, qk_heads: Optional[int] = None,
         key_norm: float = 1.0) -> Dict[str, Optional[np.ndarray]]:
    """Draw one set of per-token tensors with leading shape ``lead`` (e.g. (B, T, H)).

    Returns q, k, v, beta, wgate, g following the boundary's argument names:
    for the split-gate form ``beta`` carries the erase gate (last dim dk) and
    ``wgate`` the write gate (last dim dv); for fg2 ``beta`` is the step size
    per key channel (last dim dk); otherwise ``beta`` has shape ``lead``; and
    ``wgate`` is None except for the split-gate form.  ``g`` is None for the ungated form,
    shape ``lead`` for a scalar gate and ``lead + (dk,)`` for channel gates.
    ``gate_scale`` multiplies the log-decays (e.g. 1/16 for weak decay); channel
    log-decays are then kept at or above CHANNEL_LOG_DECAY_FLOOR.
    ``qk_heads`` replaces the last entry of ``lead`` for q and k (grouped value
    heads); ``key_norm`` is the L2 norm of every key before rounding.
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    qk_lead = lead if qk_heads is None else lead[:-1] + (qk_heads,)
    q = _unit(rng.standard_normal(qk_lead + (dk,), dtype=np.float32))
    k = _unit(rng.standard_normal(qk_lead + (dk,), dtype=np.float32))
    if key_norm != 1.0:
        k = (k * np.float32(key_norm)).astype(np.float32)
    v = rng.standard_normal(lead + (dv,), dtype=np.float32)
    if variant == "gdn2":
        beta = _sigmoid(rng.standard_normal(lead + (dk,), dtype=np.float32))
        wgate = _sigmoid(rng.standard_normal(lead + (dv,), dtype=np.float32))
    elif variant == "fg2":
        beta = _sigmoid(rng.standard_normal(lead + (dk,), dtype=np.float32))
        wgate = None
    else:
        beta = _sigmoid(rng.standard_normal(lead, dtype=np.float32))
        wgate = None
    if variant == "deltanet":
        g = None
    elif variant == "gdn":
        g = _neg_softplus(rng.standard_normal(lead, dtype=np.float32)) * np.float32(gate_scale)
    else:
        g = _neg_softplus(rng.standard_normal(lead + (dk,), dtype=np.float32)) * np.float32(gate_scale)
        g = np.maximum(g, CHANNEL_LOG_DECAY_FLOOR)
    out = dict(q=q, k=k, v=v, beta=beta, wgate=wgate, g=g)
    return {name: (None if t is None else cast(t, dtype)) for name, t in out.items()}


def make_forward_inputs(w: Workload, seed: Optional[int] = None, T: Optional[int] = None,
                        gate_scale: float = 1.0, random_s0: Optional[bool] = None,
                        qk_heads: Optional[int] = None, key_norm: float = 1.0
                        ) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of one chunkwise forward: layout [B, T, H, d] per token, S0 [B, H, dv, dk]."""
    seed = w.seed if seed is None else seed
    T = w.T if T is None else T
    random_s0 = w.random_s0 if random_s0 is None else random_s0
    rng = np.random.Generator(np.random.PCG64(seed))
    out = draw(rng, w.variant, w.dtype, (w.B, T, w.H), w.dk, w.dv, gate_scale, qk_heads, key_norm)
    if random_s0:
        out["S0"] = (np.float32(0.02) * rng.standard_normal((w.B, w.H, w.dv, w.dk),
                                                            dtype=np.float32)).astype(np.float32)
    else:
        out["S0"] = None
    return out


def make_decode_inputs(w: Workload, n_steps: int, seed: Optional[int] = None,
                       gate_scale: float = 1.0, qk_heads: Optional[int] = None,
                       key_norm: float = 1.0) -> Dict[str, object]:
    """A random fp32 state [B, H, dv, dk] and ``n_steps`` per-step input sets [B, H, d]."""
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    S = (np.float32(0.02) * rng.standard_normal((w.B, w.H, w.dv, w.dk),
                                                dtype=np.float32)).astype(np.float32)
    steps = [draw(rng, w.variant, w.dtype, (w.B, w.H), w.dk, w.dv, gate_scale, qk_heads, key_norm)
             for _ in range(n_steps)]
    return dict(S=S, steps=steps)


def make_ttt_inputs(w: Workload, seed: Optional[int] = None, T: Optional[int] = None,
                    random_states: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of DeltaTTT-pre (two memory layers): the forward inputs of ``w``
    (q, k, v, beta1 = beta, g1 = g; "deltanet" or "gdn"), then beta2 and g2
    drawn the same way, then A0 [B, H, dv, dk] and B0 [B, H, dv, dv] as
    0.02 * z (or None)."""
    if w.variant not in ("deltanet", "gdn"):
        raise ValueError("DeltaTTT-pre takes the deltanet or gdn form")
    seed = w.seed if seed is None else seed
    T = w.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(seed))
    x = draw(rng, w.variant, w.dtype, (w.B, T, w.H), w.dk, w.dv)
    lead = (w.B, T, w.H)
    beta2 = _sigmoid(rng.standard_normal(lead, dtype=np.float32))
    g2 = None if w.variant == "deltanet" else _neg_softplus(rng.standard_normal(lead, dtype=np.float32))
    out = dict(q=x["q"], k=x["k"], v=x["v"], beta1=x["beta"], g1=x["g"],
               beta2=cast(beta2, w.dtype), g2=None if g2 is None else cast(g2, w.dtype))
    if random_states:
        out["A0"] = (np.float32(0.02) * rng.standard_normal((w.B, w.H, w.dv, w.dk), dtype=np.float32))
        out["B0"] = (np.float32(0.02) * rng.standard_normal((w.B, w.H, w.dv, w.dv), dtype=np.float32))
    else:
        out["A0"] = out["B0"] = None
    return out
