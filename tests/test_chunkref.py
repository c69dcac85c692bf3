"""The chunk algebra the prefill kernel implements equals the token-by-token oracle.

The chunkwise method reaches the sequential result exactly in exact arithmetic,
so in float64 the two agree to rounding (~1e-12) for every chunk size,
including 1 (token by token) and T (one chunk), ragged tails and all variants.
"""
import numpy as np
import pytest

from chunkref import chunk_fwd
from oracle import delta_fwd
from recurrent_memory_amd.inputs import Workload, make_forward_inputs


def _inputs(variant, T, dk=8, dv=6, B=2, H=2, seed=0, gate_scale=1.0, random_s0=True):
    w = Workload("t", variant, "f32", B=B, H=H, T=T, dk=dk, dv=dv, random_s0=random_s0, seed=seed)
    return make_forward_inputs(w, gate_scale=gate_scale)


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2", "fg2"])
@pytest.mark.parametrize("chunk", [1, 4, 16, 64, 37])
def test_chunk_equals_oracle(variant, chunk):
    x = _inputs(variant, T=37, seed=chunk)
    o_ref, S_ref = delta_fwd(variant, **x)
    o, S = chunk_fwd(variant, **x, chunk=chunk)
    scale = np.abs(o_ref).max()
    assert np.abs(o - o_ref).max() <= 1e-12 * max(scale, 1.0)
    assert np.abs(S - S_ref).max() <= 1e-12 * max(np.abs(S_ref).max(), 1.0)


@pytest.mark.parametrize("variant", ["gdn", "kda", "gdn2", "fg2"])
@pytest.mark.parametrize("T", [1, 63, 65, 100])
def test_chunk_ragged_weak_decay(variant, T):
    x = _inputs(variant, T=T, seed=T, gate_scale=1 / 16)
    o_ref, S_ref = delta_fwd(variant, **x)
    o, S = chunk_fwd(variant, **x, chunk=64)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-11)


def test_gdn2_reduces_to_kda_in_chunk_form():
    x = _inputs("kda", T=70, seed=3)
    o_kda, S_kda = chunk_fwd("kda", **x, chunk=16)
    b = np.repeat(x["beta"][..., None], x["q"].shape[-1], axis=-1)
    w = np.repeat(x["beta"][..., None], x["v"].shape[-1], axis=-1)
    o2, S2 = chunk_fwd("gdn2", **{**x, "beta": b, "wgate": w}, chunk=16)
    np.testing.assert_allclose(o2, o_kda, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S_kda, rtol=0, atol=1e-12)


def test_fg2_reduces_to_kda_in_chunk_form():
    x = _inputs("kda", T=70, seed=4)
    o_kda, S_kda = chunk_fwd("kda", **x, chunk=16)
    b = np.repeat(x["beta"][..., None], x["q"].shape[-1], axis=-1)
    o2, S2 = chunk_fwd("fg2", **{**x, "beta": b}, chunk=16)
    np.testing.assert_allclose(o2, o_kda, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S_kda, rtol=0, atol=1e-12)
