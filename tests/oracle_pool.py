"""Run the CPU oracle on every (batch, head) sequence of a workload, in a pool of
worker processes (spawned; each imports only numpy and the oracle, never torch or
the GPU library), so full-size parity tests check every head rather than a sample.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

# arguments laid out [B, H, ...] (states); every other array is [B, T, heads, ...]
STATE_KEYS = ("S0", "A0", "B0", "dS_T", "S")
MAX_WORKERS = 16


def n_workers(n_jobs: int) -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0)), n_jobs))


def head_slice(x: dict, b: int, h: int, H: int) -> dict:
    """The arguments of value head h of batch b.  Query/key tensors with fewer
    heads (grouped value heads) give the head h // (H / heads)."""
    sub = {}
    for n, a in x.items():
        if not isinstance(a, np.ndarray):
            sub[n] = a
        elif n in STATE_KEYS:
            sub[n] = np.ascontiguousarray(a[b:b + 1, h:h + 1])
        else:
            hh = h // (H // a.shape[2])
            sub[n] = np.ascontiguousarray(a[b:b + 1, :, hh:hh + 1])
    return sub


def _job(job):
    from threadpoolctl import threadpool_limits

    import oracle
    name, pos, kw = job
    with threadpool_limits(1):
        return getattr(oracle, name)(*pos, **kw)


def map_heads(name: str, x: dict, B: int, H: int, pos: tuple = ()) -> dict:
    """{(b, h): oracle.<name>(*pos, **head_slice(x, b, h, H))} for every head."""
    jobs = [(name, pos, head_slice(x, b, h, H)) for b in range(B) for h in range(H)]
    with mp.get_context("spawn").Pool(n_workers(len(jobs))) as pool:
        res = pool.map(_job, jobs, chunksize=1)
    return {(b, h): res[b * H + h] for b in range(B) for h in range(H)}


def fwd_all_heads(variant: str, x: dict, B: int, H: int):
    """(o_ref [B, T, H, d_v], S_ref [B, H, d_v, d_k]) of oracle.delta_fwd, head by head."""
    res = map_heads("delta_fwd", x, B, H, pos=(variant,))
    o0, S0 = res[(0, 0)]
    o = np.empty((B, o0.shape[1], H, o0.shape[3]))
    S = np.empty((B, H) + S0.shape[2:])
    for (b, h), (ob, Sb) in res.items():
        o[b, :, h] = ob[0, :, 0]
        S[b, h] = Sb[0, 0]
    return o, S


def ttt_all_heads(variant: str, x: dict, B: int, H: int):
    """(o, A_T, B_T) of oracle.ttt_pre_fwd, head by head."""
    res = map_heads("ttt_pre_fwd", x, B, H, pos=(variant,))
    o0, A0, B0 = res[(0, 0)]
    o = np.empty((B, o0.shape[1], H, o0.shape[3]))
    AT = np.empty((B, H) + A0.shape[2:])
    BT = np.empty((B, H) + B0.shape[2:])
    for (b, h), (ob, Ab, Bb) in res.items():
        o[b, :, h] = ob[0, :, 0]
        AT[b, h] = Ab[0, 0]
        BT[b, h] = Bb[0, 0]
    return o, AT, BT


def bwd_all_heads(variant: str, x: dict, B: int, H: int) -> dict:
    """Gradients of oracle.delta_bwd, head by head (no grouped heads): x holds the
    forward inputs plus dO and dS_T."""
    res = map_heads("delta_bwd", x, B, H, pos=(variant,))
    out = {}
    for n, a0 in res[(0, 0)].items():
        if a0 is None:
            out[n] = None
        elif n == "dS0":
            out[n] = np.empty((B, H) + a0.shape[2:])
        else:
            out[n] = np.empty((B, a0.shape[1], H) + a0.shape[3:])
    for (b, h), r in res.items():
        for n, a in r.items():
            if a is None:
                continue
            if n == "dS0":
                out[n][b, h] = a[0, 0]
            else:
                out[n][b, :, h] = a[0, :, 0]
    return out
