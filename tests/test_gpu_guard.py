"""Guard canaries: every output of every entry point is placed inside a larger
buffer whose margins (and the output itself) are filled with a sentinel bit
pattern; after the call the margins must be untouched and no sentinel may be
left inside the output.  This catches stores past the end of an output (the
masked ragged last chunk, the 8-byte transposed output stores, the 16-byte state
stores) and outputs left partly unwritten.  The workspace gets the same margins."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import Workload, make_decode_inputs, make_forward_inputs, make_ttt_inputs

pytestmark = pytest.mark.gpu

MARGIN = 64 * 1024                       # bytes on each side
SENTINEL = {torch.bfloat16: -1, torch.float32: -1, torch.uint8: 0xA5}   # all-ones: a NaN
BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8}


class Guarded:
    """An output tensor of ``shape`` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype):
        esz = torch.tensor([], dtype=dtype).element_size()
        self.m = MARGIN // esz
        self.n = int(np.prod(shape))
        self.buf = torch.empty(self.n + 2 * self.m, dtype=dtype, device="cuda")
        self.buf.view(BITS[dtype]).fill_(SENTINEL[dtype])
        self.dtype = dtype
        self.t = self.buf[self.m:self.m + self.n].view(shape)

    def check(self, name, full=True):
        bits = self.buf.view(BITS[self.dtype])
        s = SENTINEL[self.dtype]
        lo, hi = bits[:self.m], bits[self.m + self.n:]
        assert bool((lo == s).all()), f"{name}: store before the output"
        assert bool((hi == s).all()), f"{name}: store past the end of the output"
        if full:
            inside = bits[self.m:self.m + self.n]
            assert not bool((inside == s).any()), f"{name}: part of the output left unwritten"


def _workspace(entry, variant, w, dtype_code, Hk=0):
    desc = ops.DrDesc(w.B, w.T, w.H, w.dk, w.dv, 64, ops.VARIANTS[variant], dtype_code, Hk or w.H)
    need = ops.workspace_bytes(entry, desc)
    return Guarded((max(need, 1),), torch.uint8), need


FORMS = ["deltanet", "gdn", "kda", "gdn2", "fg2"]


@pytest.mark.parametrize("variant", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_forward_writes_only_its_outputs(variant, dtype, T):
    announce("guard_fwd", variant, dtype, T)
    w = Workload("t", variant, dtype, B=2, H=3, T=T, dk=128, dv=64, random_s0=True, seed=90 + T)
    x = make_forward_inputs(w)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    o = Guarded((w.B, w.T, w.H, w.dv), tdt)
    S = Guarded((w.B, w.H, w.dv, w.dk), torch.float32)
    ws, need = _workspace("fwd", variant, w, 0 if dtype == "f32" else 1)
    ops.delta_fwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(x["beta"], dtype),
                  wgate=dev(x["wgate"], dtype), g=dev(x["g"], dtype), S0=dev(x["S0"], "f32"), o=o.t, S_T=S.t,
                  workspace=ws.t if need else None)
    torch.cuda.synchronize()
    o.check("o")
    S.check("S_T")
    ws.check("workspace", full=False)


@pytest.mark.parametrize("variant", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_writes_only_its_outputs(variant, dtype):
    announce("guard_decode", variant, dtype)
    w = Workload("t", variant, dtype, B=5, H=3, T=1, dk=128, dv=64, random_s0=True, seed=95)
    d = make_decode_inputs(w, 1)
    st = d["steps"][0]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    o = Guarded((w.B, w.H, w.dv), tdt)
    S = Guarded((w.B, w.H, w.dv, w.dk), torch.float32)
    S.t.copy_(torch.from_numpy(d["S"]).cuda())
    ops.delta_decode(variant, dev(st["q"], dtype), dev(st["k"], dtype), dev(st["v"], dtype), dev(st["beta"], dtype),
                     S.t, wgate=dev(st["wgate"], dtype), g=dev(st["g"], dtype), o=o.t)
    torch.cuda.synchronize()
    o.check("o")
    S.check("S")


@pytest.mark.parametrize("variant", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,Hk", [(1, 0), (65, 0), (200, 0), (130, 1)])
def test_backward_writes_only_its_outputs(variant, dtype, T, Hk):
    announce("guard_bwd", variant, dtype, T, Hk)
    w = Workload("t", variant, dtype, B=2, H=2, T=T, dk=128, dv=64, random_s0=True, seed=96 + T)
    x = make_forward_inputs(w, qk_heads=Hk or None)
    Hq = Hk or w.H
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(3)
    dO = dev(rng.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32), "f32").to(tdt)
    chan = variant in ("gdn2", "fg2")
    shapes = {"dq": (w.B, T, Hq, w.dk), "dk": (w.B, T, Hq, w.dk), "dv": (w.B, T, w.H, w.dv),
              "dbeta": (w.B, T, w.H, w.dk) if chan else (w.B, T, w.H)}
    if variant == "gdn2":
        shapes["dwgate"] = (w.B, T, w.H, w.dv)
    if variant != "deltanet":
        shapes["dg"] = (w.B, T, w.H) if variant == "gdn" else (w.B, T, w.H, w.dk)
    outs = {n: Guarded(s, tdt) for n, s in shapes.items()}
    outs["dS0"] = Guarded((w.B, w.H, w.dv, w.dk), torch.float32)
    ws, need = _workspace("bwd", variant, w, 0 if dtype == "f32" else 1, Hk)
    ops.delta_bwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(x["beta"], dtype),
                  dO, g=dev(x["g"], dtype), S0=dev(x["S0"], "f32"), wgate=dev(x["wgate"], dtype),
                  out={n: gd.t for n, gd in outs.items()}, workspace=ws.t)
    torch.cuda.synchronize()
    for n, gd in outs.items():
        gd.check(n)
    ws.check("workspace", full=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 65])
def test_ttt_writes_only_its_outputs(dtype, T):
    announce("guard_ttt", dtype, T)
    w = Workload("t", "gdn", dtype, B=2, H=3, T=T, dk=128, dv=64, seed=97)
    x = make_ttt_inputs(w)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    o = Guarded((w.B, w.T, w.H, w.dv), tdt)
    A = Guarded((w.B, w.H, w.dv, w.dk), torch.float32)
    Bm = Guarded((w.B, w.H, w.dv, w.dv), torch.float32)
    ws, need = _workspace("ttt_pre", "gdn", w, 0 if dtype == "f32" else 1)
    ops.ttt_pre("gdn", dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(x["beta1"], dtype),
                dev(x["beta2"], dtype), g1=dev(x["g1"], dtype), g2=dev(x["g2"], dtype),
                A0=dev(x["A0"], "f32"), B0=dev(x["B0"], "f32"), o=o.t, A_T=A.t, B_T=Bm.t, workspace=ws.t)
    torch.cuda.synchronize()
    o.check("o")
    A.check("A_T")
    Bm.check("B_T")
    ws.check("workspace", full=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_efla_writes_only_its_output(dtype):
    announce("guard_efla", dtype)
    w = Workload("t", "gdn", dtype, B=2, H=4, T=77, dk=128, dv=128, seed=98)
    x = make_forward_inputs(w, qk_heads=2)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = Guarded((w.B, w.T, w.H), tdt)
    ops.efla_beta("gdn", dev(x["k"], dtype), dev(x["beta"], dtype), out=out.t)
    torch.cuda.synchronize()
    out.check("beta_eff")
