#!/usr/bin/env python3
"""Benchmark of the chunkwise gated delta-rule forward (and the decode step) on one MI355X.

One bench step = one ``delta_fwd`` over the Gated DeltaNet workload
(bf16 inputs, fp32 state; B=4, H=16, T=4096, d_k=d_v=128, chunk 64, S0 = 0),
i.e. one pass of the whole chunkwise path.  ``value`` is tokens/s over the
timed region (a token carries all 16 heads), inputs already resident in HBM.
Three copies of the inputs are cycled so that no step finds its operands in
the 256 MB last-level cache left behind by the previous step.

The JSON line also carries
  roofline      the prefill kernel's algorithmic HBM bytes per launch over its
                average HIP-event duration, against 8 TB/s;
  mfma          algorithmic flops per launch over the same duration, against the
                2.5 PFLOP/s dense bf16 MFMA peak;
  decode        the single-token decode step (batch 256, 16 heads, d=128, fp32
                state updated in place), 1000 steps: state bytes moved per step
                over the per-step time, against 8 TB/s;
  cpu_baseline  the float64 CPU oracle timed on this host on the same workload
                (a process pool over (batch, head) sequences).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
PREFILL_KERNEL = "prefill_pipe_kernel"
DECODE_KERNEL = "decode_kernel"


def prefill_bytes(variant, B, T, H, dk, dv, elem=2, with_state_in=False, with_state_out=True,
                  Hk=None):
    """Algorithmic HBM bytes of one forward: every per-token input read once, o
    written once, the fp32 initial state read and the final state written once.
    With Hk query/key heads (grouped value heads) q and k count Hk heads."""
    Hk = H if Hk is None else Hk
    per_head = {"deltanet": dv + 1, "gdn": dv + 2, "kda": dk + dv + 1,
                "gdn2": 2 * dk + 2 * dv, "fg2": 2 * dk + dv}[variant] + dv      # v, gates, o
    state = 4 * dv * dk * (int(with_state_in) + int(with_state_out))
    return B * T * elem * (H * per_head + Hk * 2 * dk) + B * H * state


def bwd_bytes(variant, B, T, H, dk, dv, elem=2):
    """Algorithmic HBM bytes of one backward: the forward inputs and dO read once,
    every gradient written once, the fp32 dS_T read and dS0 written once."""
    gate = {"deltanet": 0, "gdn": 1, "kda": dk}[variant]
    per_tok = 2 * dk + dv + 1 + gate + dv          # q, k, v, beta, g, dO
    per_tok += 2 * dk + dv + 1 + gate              # dq, dk, dv, dbeta, dg
    return B * T * H * elem * per_tok + B * H * 4 * dv * dk * 3


def bwd_flops(B, T, H, dk, dv, C=64):
    """Algorithmic flops of the chunkwise backward (the forward recomputed once plus
    its reverse): 3x the forward's per-token count."""
    return 3 * (B * T * H * (6 * dk * dv + 3 * C * dk + 2 * C * dv + C * C / 3.0))


def efla_bytes(B, T, H, Hk, dk, elem=2):
    """Exact-flow step sizes: k read once, beta read and beta_eff written once."""
    return B * T * elem * (Hk * dk + 2 * H)


def prefill_flops(variant, B, T, H, dk, dv, C=64):
    """Algorithmic flops of one forward with chunk length C (triangular blocks
    counted once): 6 dk dv + 3 C dk + 2 C dv + C^2/3 per token and head for one
    step size (FG^2-GDN counted the same way), 8 dk dv + 5 C dk + 4 C dv + C^2/3
    for split gates."""
    if variant == "gdn2":
        per = 8 * dk * dv + 5 * C * dk + 4 * C * dv + C * C / 3.0
    else:
        per = 6 * dk * dv + 3 * C * dk + 2 * C * dv + C * C / 3.0
    return B * T * H * per


def prefill_flops_dense(variant, B, T, H, dk, dv, C=64):
    """Flops the chunk products issue with every C x C tile dense (no triangular
    tile skipped): 6 dk dv + 6 C dk + 4 C dv + C^2/3 per token and head (split
    gates: 8 dk dv + 10 C dk + 8 C dv + C^2/3)."""
    if variant == "gdn2":
        per = 8 * dk * dv + 10 * C * dk + 8 * C * dv + C * C / 3.0
    else:
        per = 6 * dk * dv + 6 * C * dk + 4 * C * dv + C * C / 3.0
    return B * T * H * per


def decode_bytes(B, H, dk, dv, elem=2):
    """Per decode step: the fp32 state read and written once, plus q, k, v, beta, g
    read and o written."""
    return B * H * (2 * 4 * dv * dk + elem * (2 * dk + dv + 2) + elem * dv)


KERNEL_SOURCES = {"prefill.hip": ["prefill.hip", "chunk_ops.h", "common.h"],
                  "prefill_pipe.hip": ["prefill_pipe.hip", "chunk_ops.h", "common.h"],
                  "prefill_cw.hip": ["prefill_cw.hip", "chunk_ops.h", "common.h"],
                  "decode.hip": ["decode.hip", "common.h"]}


def kernel_source_sha(name):
    """Hash of a kernel's source files (the kernel file and the headers it uses)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        h.update(open(os.path.join(ROOT, "recurrent_memory_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(record, source):
    """HBM bytes per launch from a committed rocprofv3 counter record
    (profiles/*.json: FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a reference
    copy), or None when the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_worker(args):
    from threadpoolctl import threadpool_limits
    from oracle import delta_fwd
    variant, x = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        o, S = delta_fwd(variant, **x)
        return time.perf_counter() - t0, o, S


def _head_groups(x, B, H, T, groups):
    """Split the inputs into ``groups`` jobs of whole (batch, head) sequences
    (first T tokens), [len, T, 1, ...] each; returns (jobs, pairs per job)."""
    pairs = [(b, h) for b in range(B) for h in range(H)]
    parts = [pairs[i::groups] for i in range(groups)]
    jobs = []
    for grp in parts:
        bs = [p[0] for p in grp]
        hs = [p[1] for p in grp]
        sub = {}
        for n, a in x.items():
            if a is None:
                sub[n] = None
            elif n == "S0":
                sub[n] = np.ascontiguousarray(a[bs, hs][:, None])
            else:  # [B, T, heads, ...] -> [len(grp), T, 1, ...]
                hh = [h // (H // a.shape[2]) for h in hs]
                sub[n] = np.ascontiguousarray(a[bs, :T, hh][:, :, None])
        jobs.append(sub)
    return jobs, parts


def oracle_all_heads(variant, x, B, T, H, workers):
    """The float64 oracle over every (batch, head) sequence (first T tokens) in a
    pool of ``workers`` processes, one BLAS thread each.  Returns (wall seconds
    including worker start-up, o [B, T, H, dv], S_T [B, H, dv, dk])."""
    import multiprocessing as mp
    jobs, parts = _head_groups(x, B, H, T, workers)
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(variant, j) for j in jobs])
    wall = time.perf_counter() - t0
    o = S = None
    for grp, (_, og, Sg) in zip(parts, res):
        if o is None:
            o = np.empty((B, T, H, og.shape[3]))
            S = np.empty((B, H) + Sg.shape[2:])
        for i, (b, h) in enumerate(grp):
            o[b, :, h] = og[i, :, 0]
            S[b, h] = Sg[i, 0]
    return wall, o, S


def max_rel_err(x, ref, head_axes):
    """Max over (batch, head) slices of max|x - ref| / max|ref| (the parity metric)."""
    x = np.asarray(x, np.float64)
    axes = tuple(a for a in range(x.ndim) if a not in head_axes)
    den = np.abs(ref).max(axis=axes)
    return float((np.abs(x - ref).max(axis=axes) / np.where(den == 0, 1.0, den)).max())


def cpu_baseline(variant, x, B, T, H, gpu_out, max_workers=16):
    """Time the float64 oracle on this host over every (batch, head) sequence of
    the workload (first ``T`` tokens), in a process pool, and once on a single
    core for one sequence; check the GPU outputs against it (parity metric)."""
    from threadpoolctl import threadpool_limits
    from oracle import delta_fwd
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(max_workers, host_cores, B * H))
    # one core: the first (batch, head) sequence in this process
    first = {n: (None if a is None else (a[:1, :1] if n == "S0" else a[:1, :T, :1])) for n, a in x.items()}
    with threadpool_limits(1):
        t0 = time.perf_counter()
        delta_fwd(variant, **first)
        one = time.perf_counter() - t0
    wall, o_ref, S_ref = oracle_all_heads(variant, x, B, T, H, workers)
    o, S = gpu_out
    return dict(value=B * T / wall, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"float64 token-by-token oracle over all {B}x{H} (batch, head) sequences, "
                       f"first {T} tokens each, {workers} worker processes (1 BLAS thread each), "
                       f"wall {wall:.2f} s including worker start-up",
                wall_s=wall, host_cores=host_cores,
                one_core={"tokens_per_s": T / one / H, "seconds_per_sequence": one,
                          "sample": f"one (batch, head) sequence of {T} tokens, one process, "
                                    f"one BLAS thread; a token carries all {H} heads, so "
                                    f"tokens/s = T / (H x seconds per sequence)"},
                parity={"o": max_rel_err(o[:, :T], o_ref, (0, 2)),
                        "S_T": max_rel_err(S, S_ref, (0, 1)) if T == o.shape[1] else None,
                        "metric": "max over (batch, head) of max|gpu - oracle| / max|oracle|",
                        "heads_checked": B * H})


def time_forward(w, steps, warmup, n_sets, stream, qk_heads=None):
    """Time delta_fwd on workload ``w`` with ``n_sets`` input copies cycled.

    The ``steps`` launches go back to back under ONE HIP-event span on the launch
    stream: an event recorded between two launches costs about 10 us of GPU time
    on this stack (a marker packet between the kernels), which per-launch events
    would add to every launch.  Returns (mean seconds per launch from the event
    span, wall seconds for the timed steps between two synchronizes, inputs)."""
    import torch
    from recurrent_memory_amd import ops
    from recurrent_memory_amd.inputs import make_forward_inputs
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    dev = torch.device("cuda:0")
    x = make_forward_inputs(w, qk_heads=qk_heads)

    def up(a, d=dt):
        return None if a is None else torch.from_numpy(a).to(d).to(dev)

    sets = []
    for _ in range(n_sets):
        sets.append(dict(q=up(x["q"]), k=up(x["k"]), v=up(x["v"]), beta=up(x["beta"]),
                         wgate=up(x["wgate"]), g=up(x["g"]), S0=up(x["S0"], torch.float32),
                         o=torch.empty((w.B, w.T, w.H, w.dv), dtype=dt, device=dev),
                         ST=torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)))

    def step(s):
        ops.delta_fwd(w.variant, s["q"], s["k"], s["v"], s["beta"], wgate=s["wgate"], g=s["g"],
                      S0=s["S0"], o=s["o"], S_T=s["ST"], stream=stream)

    for i in range(warmup):
        step(sets[i % n_sets])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(sets[i % n_sets])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out = (sets[0]["o"].float().cpu().numpy(), sets[0]["ST"].cpu().numpy())
    return e0.elapsed_time(e1) / 1e3 / steps, wall, x, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the non-headline forward workloads")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens per sequence in the oracle's timed sample")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB "
                         "(reference kernel for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py runs on exactly one GPU: the path shards by "
                                   "(batch, head) with no communication, but no multi-GPU run is "
                                   "part of it; use --gpus 1"}))
        sys.exit(2)

    import torch
    from recurrent_memory_amd import ops
    from recurrent_memory_amd.inputs import DECODE_HEADLINE, PREFILL_HEADLINE, WORKLOADS, \
        make_decode_inputs, make_forward_inputs

    ops.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[PREFILL_HEADLINE]
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    bf = torch.bfloat16
    stream = torch.cuda.current_stream()

    def up(a):
        return None if a is None else torch.from_numpy(a).to(bf).to(dev)

    n_sets = 3
    kern_avg_s, wall, x, gpu_out = time_forward(w, args.steps, args.warmup, n_sets, stream)
    ms_per_step = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens / (wall / args.steps)
    nbytes = prefill_bytes("gdn", B, T, H, dk, dv)
    nflops = prefill_flops("gdn", B, T, H, dk, dv)
    gbs = nbytes / kern_avg_s / 1e9
    tflops = nflops / kern_avg_s / 1e12

    result = {
        "metric": "tokens/s + % MFMA peak, GDN fwd bf16 H=16 d=128 T=4096; decode HBM GB/s",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N), "
                "g=-softplus(N))",
        "config": {"workload": "gated delta-rule chunkwise forward, scalar decay (GDN)",
                   "B": B, "H": H, "T": T, "d_k": dk, "d_v": dv, "chunk": 64,
                   "inputs": "bf16", "state": "fp32", "S0": "zero", "S_T": "written",
                   "input_sets_cycled": n_sets},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("prefill_gdn_bf16_b4_h16_t4096_d128.counters.json",
                                                 "prefill_pipe.hip"),
                     "kernel": PREFILL_KERNEL, "kernel_avg_us": kern_avg_s * 1e6,
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_launch": nflops,
                 "dense_tile_achieved": prefill_flops_dense("gdn", B, T, H, dk, dv) / kern_avg_s / 1e12,
                 "dense_tile_frac": prefill_flops_dense("gdn", B, T, H, dk, dv) / kern_avg_s / 1e12
                 / MFMA_BF16_PEAK_TFLOPS,
                 "dense_tile_flops_per_launch": prefill_flops_dense("gdn", B, T, H, dk, dv)},
    }

    if not args.no_other:
        # the other forward workloads: parity-test shapes, reported beside the headline
        others = []
        other_out = {}
        for name, sub_c, form in [("deltanet_fp32_t256_d64", 16, None),
                                  ("kda_bf16_b2_h16_t8192_d128", 32, None),
                                  ("gdn2_bf16_b1_h16_t32768_d128", 32, None),
                                  ("kda_bf16_b2_h16_t8192_d128", 32, "fg2")]:
            wo = WORKLOADS[name]
            if form is not None:   # another form on the same shape and seed
                wo = dataclasses.replace(wo, variant=form)
                name = name.replace(name.split("_")[0], form, 1)
            t_s, _, xo, oo = time_forward(wo, 5, 2, 2, stream)
            other_out[name] = (wo, xo, oo)
            elem = 4 if wo.dtype == "f32" else 2
            nb = prefill_bytes(wo.variant, wo.B, wo.T, wo.H, wo.dk, wo.dv, elem=elem,
                               with_state_in=wo.random_s0)
            chunk = 64 if wo.variant in ("deltanet", "gdn") else sub_c
            nf = prefill_flops(wo.variant, wo.B, wo.T, wo.H, wo.dk, wo.dv, C=chunk)
            others.append({"workload": name, "variant": wo.variant, "dtype": wo.dtype,
                           "kernel_avg_us": t_s * 1e6, "tokens_per_s": wo.B * wo.T / t_s,
                           "hbm_GBs": nb / t_s / 1e9, "hbm_frac": nb / t_s / 1e9 / HBM_PEAK_GBS,
                           "tflops": nf / t_s / 1e12, "flops_chunk_length": chunk,
                           "tflops_dense_tile": prefill_flops_dense(wo.variant, wo.B, wo.T, wo.H, wo.dk,
                                                                    wo.dv, C=chunk) / t_s / 1e12,
                           "algorithmic_bytes_per_launch": nb})
        # grouped value heads: the headline shape with 8 query/key heads (pairs of value heads)
        t_s, _, xg, og = time_forward(w, 5, 2, 2, stream, qk_heads=8)
        other_out["gdn_bf16_b4_h16_t4096_d128_hk8"] = (w, xg, og)
        nb = prefill_bytes("gdn", B, T, H, dk, dv, Hk=8)
        others.append({"workload": "gdn_bf16_b4_h16_t4096_d128_hk8", "variant": "gdn",
                       "dtype": "bf16", "qk_heads": 8, "kernel_avg_us": t_s * 1e6,
                       "tokens_per_s": B * T / t_s, "hbm_GBs": nb / t_s / 1e9,
                       "hbm_frac": nb / t_s / 1e9 / HBM_PEAK_GBS,
                       "tflops": nflops / t_s / 1e12, "algorithmic_bytes_per_launch": nb})
        # exact-flow step sizes on the headline shape (an HBM-bound pass over k)
        xe = make_forward_inputs(w)
        esets = [(up(xe["k"]), up(xe["beta"]), torch.empty((B, T, H), dtype=bf, device=dev))
                 for _ in range(3)]
        for i in range(3):
            ops.efla_beta("gdn", *esets[i][:2], out=esets[i][2], stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(30):
            ops.efla_beta("gdn", *esets[i % 3][:2], out=esets[i % 3][2], stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_e = e0.elapsed_time(e1) / 1e3 / 30
        nb = efla_bytes(B, T, H, H, dk)
        others.append({"workload": "efla_beta_bf16_b4_h16_t4096_d128", "kernel": "efla_beta_kernel",
                       "kernel_avg_us": t_e * 1e6, "hbm_GBs": nb / t_e / 1e9,
                       "hbm_frac": nb / t_e / 1e9 / HBM_PEAK_GBS,
                       "algorithmic_bytes_per_launch": nb})
        # backward of the headline forward
        xb = make_forward_inputs(w)
        bsets = []
        for _ in range(2):
            bsets.append([up(xb[n]) for n in ("q", "k", "v", "beta", "g")] +
                         [torch.randn((B, T, H, dv), device=dev).to(bf)])
        ops.delta_bwd("gdn", *bsets[0][:4], bsets[0][5], g=bsets[0][4], stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(4):
            bs = bsets[i % 2]
            ops.delta_bwd("gdn", *bs[:4], bs[5], g=bs[4], stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_b = e0.elapsed_time(e1) / 1e3 / 4
        nb, nf = bwd_bytes("gdn", B, T, H, dk, dv), bwd_flops(B, T, H, dk, dv)
        others.append({"workload": "gdn_bwd_bf16_b4_h16_t4096_d128", "kernel": "bwd_* (4 launches)",
                       "kernel_avg_us": t_b * 1e6, "tokens_per_s": B * T / t_b,
                       "hbm_GBs": nb / t_b / 1e9, "hbm_frac": nb / t_b / 1e9 / HBM_PEAK_GBS,
                       "tflops": nf / t_b / 1e12, "algorithmic_bytes_per_launch": nb,
                       "algorithmic_flops_per_launch": nf,
                       "workspace_bytes": ops.workspace_bytes(
                           "bwd", ops.DrDesc(B, T, H, dk, dv, 64, ops.VARIANTS["gdn"], ops.DTYPES[bf], H))})
        # DeltaTTT-pre (two memory layers) on the headline shape
        from recurrent_memory_amd.inputs import make_ttt_inputs
        xt = make_ttt_inputs(w)
        tsets = []
        for _ in range(2):
            tsets.append({n: (None if a is None else (torch.from_numpy(a).to(dev) if n in ("A0", "B0") else up(a)))
                          for n, a in xt.items()})

        def ttt_call(ts):
            return ops.ttt_pre("gdn", ts["q"], ts["k"], ts["v"], ts["beta1"], ts["beta2"], g1=ts["g1"],
                               g2=ts["g2"], A0=ts["A0"], B0=ts["B0"], stream=stream)
        ttt_call(tsets[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(10):
            ttt_call(tsets[i % 2])
        e1.record(stream)
        torch.cuda.synchronize()
        t_t = e0.elapsed_time(e1) / 1e3 / 10
        # algorithmic bytes: q, k, v, beta1, g1, beta2, g2 read, o written, both states in and out
        nb = B * T * H * 2 * (2 * dk + 2 * dv + 4) + B * H * 4 * (dv * dk + dv * dv) * 2
        others.append({"workload": "ttt_pre_gdn_bf16_b4_h16_t4096_d128", "kernel": "delta_ttt_pre (6 launches)",
                       "kernel_avg_us": t_t * 1e6, "tokens_per_s": B * T / t_t,
                       "hbm_GBs": nb / t_t / 1e9, "hbm_frac": nb / t_t / 1e9 / HBM_PEAK_GBS,
                       "algorithmic_bytes_per_launch": nb})
        result["other_workloads"] = others

    if not args.no_decode:
        wd = WORKLOADS[DECODE_HEADLINE]
        n_distinct = 16
        d = make_decode_inputs(wd, n_distinct)
        S = torch.from_numpy(d["S"]).to(dev)
        steps_in = [{n: up(a) for n, a in s.items()} for s in d["steps"]]
        od = torch.empty((wd.B, wd.H, wd.dv), dtype=bf, device=dev)

        def dstep(i):
            s = steps_in[i % n_distinct]
            ops.delta_decode("gdn", s["q"], s["k"], s["v"], s["beta"], S, g=s["g"], o=od,
                             stream=stream)

        for i in range(10):
            dstep(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            dstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        dstep_s = e0.elapsed_time(e1) / 1e3 / args.decode_steps
        dbytes = decode_bytes(wd.B, wd.H, wd.dk, wd.dv)
        result["decode"] = {
            "workload": "gated delta-rule decode step, scalar decay, batch 256, H=16, d=128, "
                        "fp32 state in place",
            "steps": args.decode_steps, "us_per_step": dstep_s * 1e6,
            "achieved": dbytes / dstep_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dbytes / dstep_s / 1e9 / HBM_PEAK_GBS, "bytes_per_step": dbytes,
            "traffic": measured_traffic("decode_gdn_bf16_b256_h16_d128.counters.json", "decode.hip"),
            "kernel": DECODE_KERNEL, "step_inputs_cycled": n_distinct}

    if args.calib_copy_mib > 0:
        # reference copy of known size; a 1 GiB fill in between evicts the
        # source from the 256 MB last-level cache so its reads reach HBM
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        flush = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev)
        flush.fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n * 4

    if not args.no_cpu_baseline:
        Tc = min(args.cpu_tokens, T)
        result["cpu_baseline"] = cpu_baseline("gdn", x, B, Tc, H, gpu_out)
        if not args.no_other:
            # parity of the other forward workloads on every (batch, head), same metric
            workers = result["cpu_baseline"]["cores"]
            for o_rec in result["other_workloads"]:
                name = o_rec["workload"]
                if name not in other_out:
                    continue
                wo, xo, (og, Sg) = other_out[name]
                _, o_ref, S_ref = oracle_all_heads(wo.variant, xo, wo.B, wo.T, wo.H, workers)
                o_rec["parity"] = {"o": max_rel_err(og, o_ref, (0, 2)), "S_T": max_rel_err(Sg, S_ref, (0, 1)),
                                   "heads_checked": wo.B * wo.H}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
