"""C ABI contract on the CPU: the library loads, exports what the header declares,
and rejects bad arguments with the documented status before any HIP call.

Every call here fails validation, so no pointer is ever dereferenced (the
pointers are fake, aligned, non-overlapping addresses) and nothing is launched.
"""
import ctypes

import pytest

from recurrent_memory_amd import ops

lib = ops.load_library()

(DR_OK, DR_E_NULLPTR, DR_E_SHAPE, DR_E_UNSUPPORTED, DR_E_ALIGN, DR_E_DEVICE, DR_E_LAUNCH, DR_E_ALIAS,
 DR_E_WORKSPACE) = range(9)
FAKE = [ctypes.c_void_p(0x7f0000000000 + (i << 32)) for i in range(16)]
WS = FAKE[15]          # a fake 256-byte aligned workspace, far from every tensor
WS_BYTES = 1 << 31


def test_exports_every_header_symbol():
    names = ops.header_functions()
    assert set(names) == {"delta_fwd", "delta_decode", "delta_bwd", "delta_efla_beta",
                          "delta_ttt_pre", "dr_status_str", "dr_abi_version",
                          "delta_fwd_workspace_bytes", "delta_bwd_workspace_bytes",
                          "delta_ttt_pre_workspace_bytes", "delta_fwd_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert lib.dr_abi_version() == ops.ABI_VERSION == 5
    assert lib.dr_status_str(0) == b"ok"
    assert lib.dr_status_str(99) == b"unknown status"
    for s in range(9):
        assert lib.dr_status_str(s) and lib.dr_status_str(s) != b"unknown status"


def desc(**kw):
    d = dict(B=2, T=100, H=3, d_k=128, d_v=128, chunk=64, variant=1, dtype=1)
    d.update(kw)
    return ops.DrDesc(**d)


def fwd(d, q=FAKE[0], k=FAKE[1], v=FAKE[2], beta=FAKE[3], wgate=None, g=FAKE[5], S0=None,
        o=FAKE[7], ST=None, ws=WS, ws_bytes=WS_BYTES):
    return lib.delta_fwd(ctypes.byref(d) if d is not None else None, q, k, v, beta, wgate, g, S0,
                         o, ST, ws, ws_bytes, None)


def dec(d, q=FAKE[0], k=FAKE[1], v=FAKE[2], beta=FAKE[3], wgate=None, g=FAKE[5], S=FAKE[6],
        o=FAKE[7]):
    return lib.delta_decode(ctypes.byref(d) if d is not None else None, q, k, v, beta, wgate, g,
                            S, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(variant=5), DR_E_UNSUPPORTED), (dict(variant=-1), DR_E_UNSUPPORTED),
    (dict(dtype=2), DR_E_UNSUPPORTED), (dict(d_k=96), DR_E_UNSUPPORTED),
    (dict(d_v=256), DR_E_UNSUPPORTED), (dict(chunk=32), DR_E_UNSUPPORTED),
    (dict(B=0), DR_E_SHAPE), (dict(T=0), DR_E_SHAPE), (dict(H=-1), DR_E_SHAPE),
    (dict(T=1 << 30, B=1 << 10), DR_E_SHAPE),
    # grid and 32-bit offset limits: B*H <= 2^20, B*H*ceil(T/64) <= 2^22, H < 2^18
    (dict(B=1 << 18, H=5, T=1), DR_E_SHAPE), (dict(B=1 << 10, H=1 << 6, T=65 * 64), DR_E_SHAPE),
    (dict(B=1, H=1 << 18, T=1), DR_E_SHAPE),
    (dict(H_k=2), DR_E_SHAPE), (dict(H_k=4), DR_E_SHAPE), (dict(H_k=-1), DR_E_SHAPE),
])
def test_bad_descriptor(kw, status):
    assert fwd(desc(**kw)) == status


def test_null_descriptor_and_pointers():
    assert fwd(None) == DR_E_NULLPTR
    assert dec(None) == DR_E_NULLPTR
    for name in ("q", "k", "v", "beta", "o"):
        assert fwd(desc(), **{name: None}) == DR_E_NULLPTR, name
    assert fwd(desc(variant=1), g=None) == DR_E_NULLPTR
    assert fwd(desc(variant=3), wgate=None) == DR_E_NULLPTR
    assert dec(desc(T=1), S=None) == DR_E_NULLPTR


def test_arguments_the_variant_does_not_take():
    assert fwd(desc(variant=0)) == DR_E_UNSUPPORTED            # decay given to the ungated form
    assert fwd(desc(variant=1), wgate=FAKE[4]) == DR_E_UNSUPPORTED
    assert fwd(desc(variant=4), wgate=FAKE[4]) == DR_E_UNSUPPORTED   # FG^2-GDN has no write gate
    assert dec(desc(variant=4, T=1), wgate=FAKE[4]) == DR_E_UNSUPPORTED


def test_channel_step_sizes_are_sized_per_key_channel():
    """For FG^2-GDN beta spans B*T*H*d_k elements: an output over its last 16 bytes
    is rejected (it would lie past beta with one step size per token)."""
    d = desc(variant=4, T=64, B=1)
    inside = ctypes.c_void_p(FAKE[3].value + 1 * 64 * 3 * 128 * 2 - 16)
    assert fwd(d, o=inside) == DR_E_ALIAS
    inside_scalar = ctypes.c_void_p(FAKE[3].value + 1 * 64 * 3 * 2 - 16)
    assert fwd(desc(variant=2, T=64, B=1), o=inside_scalar) == DR_E_ALIAS


def test_alignment():
    bad = ctypes.c_void_p(FAKE[0].value + 8)
    assert fwd(desc(), q=bad) == DR_E_ALIGN
    assert fwd(desc(), S0=ctypes.c_void_p(FAKE[8].value + 4)) == DR_E_ALIGN
    assert dec(desc(T=1), S=ctypes.c_void_p(FAKE[6].value + 4)) == DR_E_ALIGN


def test_aliasing():
    assert fwd(desc(), o=FAKE[2]) == DR_E_ALIAS                 # o == v
    assert fwd(desc(), ST=FAKE[0]) == DR_E_ALIAS                # S_T == q
    inside = ctypes.c_void_p(FAKE[8].value + 256)
    assert fwd(desc(), S0=FAKE[8], ST=inside) == DR_E_ALIAS     # partial overlap with S0
    assert dec(desc(T=1), o=FAKE[6]) == DR_E_ALIAS              # o == S
    assert dec(desc(T=1), S=FAKE[0]) == DR_E_ALIAS              # S == q


def efla(d, k=FAKE[1], beta=FAKE[3], out=FAKE[9]):
    return lib.delta_efla_beta(ctypes.byref(d) if d is not None else None, k, beta, out, None)


def test_efla_validation():
    assert efla(None) == DR_E_NULLPTR
    assert efla(desc(), k=None) == DR_E_NULLPTR
    assert efla(desc(), out=None) == DR_E_NULLPTR
    assert efla(desc(variant=3)) == DR_E_UNSUPPORTED            # split gates have no single step
    assert efla(desc(variant=4)) == DR_E_UNSUPPORTED            # nor do per-channel step sizes
    assert efla(desc(H_k=2)) == DR_E_SHAPE
    assert efla(desc(), beta=ctypes.c_void_p(FAKE[3].value + 2)) == DR_E_ALIGN
    assert efla(desc(), out=FAKE[1]) == DR_E_ALIAS              # beta_eff over k
    assert efla(desc(), out=ctypes.c_void_p(FAKE[3].value + 16)) == DR_E_ALIAS  # shifted onto beta


def test_grouped_heads_size_the_query_key_operands():
    """With H_k query/key heads, q and k span B*T*H_k*d_k elements: an output
    over the last 16 bytes of k is rejected, one right after k is accepted (it
    would lie inside k if k were sized with H heads)."""
    d = desc(H=4, H_k=2, T=64, B=1)
    qk_bytes = 1 * 64 * 2 * 128 * 2
    after_k = ctypes.c_void_p(FAKE[1].value + qk_bytes)
    inside_ungrouped = ctypes.c_void_p(FAKE[1].value + qk_bytes - 16)
    assert fwd(d, o=inside_ungrouped) == DR_E_ALIAS
    import torch
    if not torch.cuda.is_available():
        assert fwd(d, o=after_k) == DR_E_DEVICE


def bwd(d, q=FAKE[0], k=FAKE[1], v=FAKE[2], beta=FAKE[3], wgate=None, g=FAKE[5], S0=None,
        dO=FAKE[4], dST=None, dq=FAKE[7], dk=FAKE[8], dv=FAKE[9], dbeta=FAKE[10], dwgate=None,
        dg=FAKE[11], dS0=None, ws=WS, ws_bytes=WS_BYTES):
    return lib.delta_bwd(ctypes.byref(d) if d is not None else None, q, k, v, beta, wgate, g, S0,
                         dO, dST, dq, dk, dv, dbeta, dwgate, dg, dS0, ws, ws_bytes, None)


def test_bwd_validation():
    assert bwd(None) == DR_E_NULLPTR
    for name in ("q", "k", "v", "beta", "dO", "dq", "dk", "dv", "dbeta"):
        assert bwd(desc(), **{name: None}) == DR_E_NULLPTR, name
    assert bwd(desc(variant=1), g=None) == DR_E_NULLPTR
    assert bwd(desc(variant=1), dg=None) == DR_E_NULLPTR
    assert bwd(desc(variant=0), g=None) == DR_E_UNSUPPORTED     # dg given to the ungated form
    assert bwd(desc(variant=3)) == DR_E_NULLPTR                 # split gates need the write gate
    assert bwd(desc(variant=3), wgate=FAKE[6]) == DR_E_NULLPTR  # ... and its gradient
    assert bwd(desc(variant=1), dwgate=FAKE[6]) == DR_E_UNSUPPORTED
    assert bwd(desc(variant=4), wgate=FAKE[6]) == DR_E_UNSUPPORTED   # FG^2-GDN has no write gate
    assert bwd(desc(), dq=FAKE[0]) == DR_E_ALIAS                # dq over q
    assert bwd(desc(), dv=FAKE[8]) == DR_E_ALIAS                # dv over dk
    assert bwd(desc(), dS0=ctypes.c_void_p(FAKE[6].value + 4)) == DR_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert bwd(desc()) == DR_E_DEVICE
        assert bwd(desc(variant=0), g=None, dg=None) == DR_E_DEVICE


def test_decode_requires_one_token():
    assert dec(desc(T=2)) == DR_E_SHAPE


def test_no_device_returns_device_error():
    """With valid arguments and no usable GPU the call reports DR_E_DEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid arguments would launch on fake pointers")
    assert fwd(desc(), S0=FAKE[8], ST=FAKE[8]) == DR_E_DEVICE
    assert dec(desc(T=1)) == DR_E_DEVICE
    assert efla(desc(T=1)) == DR_E_DEVICE
    assert efla(desc(), out=FAKE[3]) == DR_E_DEVICE             # in place is allowed


def ttt(d, q=FAKE[0], k=FAKE[1], v=FAKE[2], beta1=FAKE[3], g1=FAKE[4], beta2=FAKE[5], g2=FAKE[6],
        A0=None, B0=None, o=FAKE[9], AT=None, BT=None, ws=WS, ws_bytes=WS_BYTES):
    return lib.delta_ttt_pre(ctypes.byref(d) if d is not None else None, q, k, v, beta1, g1, beta2, g2,
                             A0, B0, o, AT, BT, ws, ws_bytes, None)


def test_ttt_pre_validation():
    assert ttt(None) == DR_E_NULLPTR
    for name in ("q", "k", "v", "beta1", "beta2", "o", "g1", "g2"):
        assert ttt(desc(), **{name: None}) == DR_E_NULLPTR, name
    assert ttt(desc(variant=0)) == DR_E_UNSUPPORTED             # decays given to the ungated form
    for var in (2, 3, 4):
        assert ttt(desc(variant=var)) == DR_E_UNSUPPORTED       # deltanet or gdn only
    assert ttt(desc(H=4, H_k=2)) == DR_E_UNSUPPORTED            # no grouped heads
    assert ttt(desc(), o=FAKE[2]) == DR_E_ALIAS                 # o over v
    assert ttt(desc(), AT=FAKE[10], BT=FAKE[10]) == DR_E_ALIAS  # the two final states overlap
    assert ttt(desc(), A0=FAKE[10], BT=FAKE[10]) == DR_E_ALIAS  # B_T over A0
    assert ttt(desc(), B0=ctypes.c_void_p(FAKE[11].value + 4)) == DR_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert ttt(desc(), A0=FAKE[10], AT=FAKE[10], B0=FAKE[11], BT=FAKE[11]) == DR_E_DEVICE  # in place
        assert ttt(desc(variant=0), g1=None, g2=None) == DR_E_DEVICE


def ws_bytes(entry, d):
    n = ctypes.c_size_t(0)
    st = getattr(lib, f"delta_{entry}_workspace_bytes")(ctypes.byref(d) if d is not None else None,
                                                        ctypes.byref(n))
    return st, n.value


def test_workspace_size_queries():
    """Sizes follow the header's statement: none for the scalar-decay forward and
    for fp32 channel-wise forms; one 38 KiB (split gates: 50 KiB) block per 32
    tokens of a head for the bf16 channel-wise forward; one record per 64 tokens
    of a head for the backward (d = 128: 272.75 KiB for the ungated and scalar-decay
    forms, 400.5 KiB for KDA and FG^2-GDN, 560.5 KiB for the split gates), plus two
    fp32 [B,T,H,d_k] buffers with grouped heads; the DeltaTTT-pre intermediates."""
    up = lambda n: (n + 255) // 256 * 256
    assert ws_bytes("fwd", None)[0] == DR_E_NULLPTR
    assert lib.delta_fwd_workspace_bytes(ctypes.byref(desc()), None) == DR_E_NULLPTR
    assert ws_bytes("fwd", desc(d_k=96))[0] == DR_E_UNSUPPORTED
    assert ws_bytes("fwd", desc(variant=1)) == (DR_OK, 0)
    assert ws_bytes("fwd", desc(variant=2, dtype=0)) == (DR_OK, 0)
    nc = (100 + 31) // 32
    assert ws_bytes("fwd", desc(variant=2)) == (DR_OK, up(2 * 3 * nc * 38 * 1024))
    assert ws_bytes("fwd", desc(variant=4)) == (DR_OK, up(2 * 3 * nc * 38 * 1024))
    assert ws_bytes("fwd", desc(variant=3)) == (DR_OK, up(2 * 3 * nc * 50 * 1024))
    assert ws_bytes("fwd", desc(variant=2, d_k=64)) == (DR_OK, up(2 * 3 * nc * 21 * 1024))
    assert ws_bytes("fwd", desc(variant=3, d_k=64)) == (DR_OK, up(2 * 3 * nc * 29 * 1024))
    n64 = (100 + 63) // 64
    assert ws_bytes("bwd", desc(variant=1)) == (DR_OK, up(2 * 3 * n64 * 27275 * 1024 // 100))
    assert ws_bytes("bwd", desc(variant=0)) == (DR_OK, up(2 * 3 * n64 * 27275 * 1024 // 100))
    assert ws_bytes("bwd", desc(variant=2)) == (DR_OK, up(2 * 3 * n64 * 4005 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=4)) == (DR_OK, up(2 * 3 * n64 * 4005 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=3)) == (DR_OK, up(2 * 3 * n64 * 5605 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=3, d_k=128, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 4645 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=3, d_k=64, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 30425 * 1024 // 100))
    assert ws_bytes("bwd", desc(variant=1, d_k=64, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 1285 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=2, d_k=64, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 19225 * 1024 // 100))
    assert ws_bytes("bwd", desc(variant=1, d_k=128, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 20875 * 1024 // 100))
    assert ws_bytes("bwd", desc(variant=2, d_k=128, d_v=64)) == (DR_OK, up(2 * 3 * n64 * 3365 * 1024 // 10))
    assert ws_bytes("bwd", desc(variant=1, d_k=64, d_v=128)) == (DR_OK, up(2 * 3 * n64 * 1925 * 1024 // 10))
    grouped = ws_bytes("bwd", desc(variant=1, H=4, H_k=2))[1]
    assert grouped == up(2 * 4 * n64 * 27275 * 1024 // 100) + 2 * up(2 * 100 * 4 * 128 * 4)
    tok = 2 * 100 * 3
    f32_pieces = up(tok * 128 * 4) + 4 * up(tok * 128 * 4) + up(2 * 3 * 128 * 4)
    assert ws_bytes("ttt_pre", desc(variant=1, dtype=0)) == (DR_OK, f32_pieces)
    # bf16: fp32 copies of q, k, v, the four per-token scalars and the output, then the fp32 pieces
    wide = 4 * up(tok * 128 * 4) + 4 * up(tok * 4)
    assert ws_bytes("ttt_pre", desc(variant=1)) == (DR_OK, wide + f32_pieces)
    assert ws_bytes("ttt_pre", desc(variant=2))[0] == DR_E_UNSUPPORTED


def test_workspace_validation():
    """A needed workspace that is missing, too small, misaligned or over a tensor
    is refused before any HIP call; one that is not needed may be NULL."""
    d = desc(variant=2)
    need = ws_bytes("fwd", d)[1]
    assert fwd(d, ws=None, ws_bytes=0) == DR_E_WORKSPACE
    assert fwd(d, ws_bytes=need - 1) == DR_E_WORKSPACE
    assert fwd(d, ws=ctypes.c_void_p(WS.value + 16)) == DR_E_ALIGN
    assert fwd(d, ws=FAKE[2]) == DR_E_ALIAS                            # over v
    assert fwd(d, ws=ctypes.c_void_p(FAKE[7].value - 256), ws_bytes=need) == DR_E_ALIAS   # runs into o
    assert bwd(desc(), ws=None, ws_bytes=0) == DR_E_WORKSPACE
    assert bwd(desc(), ws=FAKE[9]) == DR_E_ALIAS                       # over dv
    assert ttt(desc(), ws=None, ws_bytes=0) == DR_E_WORKSPACE
    assert ttt(desc(), ws=FAKE[0]) == DR_E_ALIAS                       # over q
    import torch
    if not torch.cuda.is_available():
        assert fwd(desc(variant=1), ws=None, ws_bytes=0) == DR_E_DEVICE   # none needed
        assert fwd(d, ws_bytes=need) == DR_E_DEVICE


def fwd_noalloc(d, q=FAKE[0], k=FAKE[1], v=FAKE[2], beta=FAKE[3], wgate=None, g=FAKE[5], S0=None,
                o=FAKE[7], ST=None):
    return lib.delta_fwd_noalloc(ctypes.byref(d) if d is not None else None, q, k, v, beta, wgate, g,
                                 S0, o, ST, None)


def test_noalloc_validation():
    """The entry point without a workspace validates like delta_fwd and refuses
    descriptors whose workspace would exceed its 64 MiB scratch, before any HIP call."""
    assert fwd_noalloc(None) == DR_E_NULLPTR
    assert fwd_noalloc(desc(), o=FAKE[2]) == DR_E_ALIAS
    assert fwd_noalloc(desc(d_k=96)) == DR_E_UNSUPPORTED
    assert fwd_noalloc(desc(), q=ctypes.c_void_p(FAKE[0].value + 8)) == DR_E_ALIGN
    big = desc(variant=2, B=1, H=1, T=1725 * 32)            # 1725 blocks of 38 KiB > 64 MiB
    assert ws_bytes("fwd", big)[1] > (64 << 20)
    assert fwd_noalloc(big) == DR_E_WORKSPACE
    assert ws_bytes("fwd", desc(variant=2, B=1, H=1, T=1724 * 32))[1] <= (64 << 20)
    import torch
    if not torch.cuda.is_available():
        assert fwd_noalloc(desc(variant=2, B=1, H=1, T=1724 * 32)) == DR_E_DEVICE
        assert fwd_noalloc(desc(variant=1)) == DR_E_DEVICE
