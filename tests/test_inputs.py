"""The seeded workload generator: shapes, ranges, determinism, bf16 rounding."""
import numpy as np
import torch

from recurrent_memory_amd.inputs import WORKLOADS, Workload, make_decode_inputs, \
    make_forward_inputs, make_ttt_inputs, round_to_bf16


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.3e38], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_to_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_forward_inputs_shapes_and_ranges():
    w = Workload("t", "gdn2", "bf16", B=2, H=3, T=10, dk=8, dv=4, random_s0=True, seed=5)
    x = make_forward_inputs(w)
    assert x["q"].shape == (2, 10, 3, 8) and x["v"].shape == (2, 10, 3, 4)
    assert x["beta"].shape == (2, 10, 3, 8) and x["wgate"].shape == (2, 10, 3, 4)
    assert x["g"].shape == (2, 10, 3, 8) and x["S0"].shape == (2, 3, 4, 8)
    assert (x["g"] <= 0).all() and (x["beta"] > 0).all() and (x["beta"] < 1).all()
    n = np.linalg.norm(x["q"].astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-2
    for name in ("q", "k", "v", "beta", "wgate", "g"):
        assert np.array_equal(round_to_bf16(x[name]), x[name])
    y = make_forward_inputs(w)
    assert all(np.array_equal(x[n], y[n]) for n in x)


def test_variant_layouts():
    for variant, bshape, gshape in [("deltanet", (1, 5, 2), None), ("gdn", (1, 5, 2), (1, 5, 2)),
                                    ("kda", (1, 5, 2), (1, 5, 2, 4)), ("fg2", (1, 5, 2, 4), (1, 5, 2, 4))]:
        x = make_forward_inputs(Workload("t", variant, "f32", 1, 2, 5, 4, 4, seed=1))
        assert x["beta"].shape == bshape and x["wgate"] is None and x["S0"] is None
        assert (x["g"] is None) == (gshape is None) and (gshape is None or x["g"].shape == gshape)


def test_decode_inputs():
    w = WORKLOADS["gdn_decode_bf16_b256_h16_d128"]
    small = Workload("t", "gdn", "bf16", B=3, H=2, T=1, dk=8, dv=8, random_s0=True, seed=w.seed)
    d = make_decode_inputs(small, 3)
    assert d["S"].shape == (3, 2, 8, 8) and len(d["steps"]) == 3
    assert d["steps"][0]["q"].shape == (3, 2, 8) and d["steps"][0]["g"].shape == (3, 2)


def test_ttt_inputs():
    w = Workload("t", "gdn", "bf16", B=2, H=3, T=7, dk=8, dv=4, seed=9)
    x = make_ttt_inputs(w)
    assert x["q"].shape == (2, 7, 3, 8) and x["v"].shape == (2, 7, 3, 4)
    for n in ("beta1", "beta2", "g1", "g2"):
        assert x[n].shape == (2, 7, 3)
        assert np.array_equal(round_to_bf16(x[n]), x[n])
    assert (x["beta2"] > 0).all() and (x["beta2"] < 1).all() and (x["g2"] <= 0).all()
    assert x["A0"].shape == (2, 3, 4, 8) and x["B0"].shape == (2, 3, 4, 4)
    # the first layer's inputs are the forward draw of the same seed
    f = make_forward_inputs(w)
    for a, b in (("q", "q"), ("k", "k"), ("v", "v"), ("beta1", "beta"), ("g1", "g")):
        assert np.array_equal(x[a], f[b])
    y = make_ttt_inputs(w)
    assert all(np.array_equal(x[n], y[n]) for n in x)
    z = make_ttt_inputs(Workload("t", "deltanet", "f32", B=1, H=1, T=3, dk=4, dv=4, seed=1), random_states=False)
    assert z["g1"] is None and z["g2"] is None and z["A0"] is None and z["B0"] is None
