"""C-ABI checks that need no GPU: the library loads, exports every declared
function, and rejects bad arguments on the host before any launch."""
import ctypes
import math

import pytest

import taylor_series_linear_amd as tl
from taylor_series_linear_amd import (TAYLOR_BF16, TAYLOR_ERR_BAD_SCALE, TAYLOR_ERR_BAD_SHAPE,
                                      TAYLOR_ERR_NULL_PTR, TAYLOR_ERR_UNSUPPORTED,
                                      TAYLOR_ERR_WORKSPACE, TAYLOR_F32, TAYLOR_OK)

L = tl.lib()
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_every_declared_function_is_exported():
    names = tl.header_functions()
    assert set(names) == {"taylor_feature_dim", "taylor_is_supported", "taylor_last_error",
                          "taylor_feature_map", "taylor_attn_prefill_workspace",
                          "taylor_attn_prefill", "taylor_attn_decode",
                          "taylor_attn_prefill_decayed_workspace", "taylor_attn_prefill_decayed",
                          "taylor_attn_decode_decayed", "taylor_attn_prefill_ext_workspace",
                          "taylor_attn_prefill_ext", "taylor_attn_decode_ext",
                          "taylor_attn_prefill_noalloc"}
    for n in names:
        assert hasattr(L, n), n


def test_feature_dim():
    for d, n, F in [(16, 3, 153), (16, 5, 4845), (64, 3, 2145), (16, 7, 74613), (16, 1, 1), (1, 4, 4)]:
        assert L.taylor_feature_dim(d, n) == F == math.comb(d + n - 1, n - 1)
    assert L.taylor_feature_dim(0, 3) == -1
    assert L.taylor_feature_dim(16, 0) == -1


def test_supported_set():
    ok = {(16, dv, n) for dv in (16, 64) for n in (1, 3, 5)} | {(dd, dv, n) for dd in (32, 64) for dv in (16, 64)
                                                                for n in (1, 3)} | {(16, 64, 7)}
    for d in (8, 16, 32, 64):
        for dv in (8, 16, 32, 64, 128):
            for n in range(0, 10):
                assert bool(L.taylor_is_supported(d, dv, n)) == ((d, dv, n) in ok)


def _prefill(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=TAYLOR_BF16, B=1, H=2, N=64, d=16, dv=64,
                n=3, a=4.0, S0=None, z0=None, o=FAKE, out_dtype=TAYLOR_BF16, S=None, z=None,
                ws=None, ws_bytes=0)
    args.update(kw)
    return L.taylor_attn_prefill(args["q"], args["k"], args["v"], args["in_dtype"], args["B"],
                                 args["H"], args["N"], args["d"], args["dv"], args["n"], args["a"],
                                 args["S0"], args["z0"], args["o"], args["out_dtype"], args["S"],
                                 args["z"], args["ws"], args["ws_bytes"], None)


def test_prefill_rejects_bad_arguments():
    assert _prefill(n=2) == TAYLOR_ERR_UNSUPPORTED
    assert b"odd" in L.taylor_last_error()
    assert _prefill(n=4) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(d=48) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(d=32, n=5) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(dv=32) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(d=64, n=5) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(in_dtype=7) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(out_dtype=9) == TAYLOR_ERR_UNSUPPORTED
    assert _prefill(B=-1) == TAYLOR_ERR_BAD_SHAPE
    assert _prefill(N=-5) == TAYLOR_ERR_BAD_SHAPE
    assert _prefill(B=1 << 20, H=1 << 20, N=1 << 20) == TAYLOR_ERR_BAD_SHAPE
    for a in (0.0, -1.0, float("nan"), float("inf")):
        assert _prefill(a=a) == TAYLOR_ERR_BAD_SCALE
    assert _prefill(q=None) == TAYLOR_ERR_NULL_PTR
    assert _prefill(S0=FAKE) == TAYLOR_ERR_NULL_PTR
    assert _prefill(z=FAKE) == TAYLOR_ERR_NULL_PTR
    need = L.taylor_attn_prefill_workspace(1, 2, 64, 16, 64, 3, TAYLOR_BF16)
    assert need != ctypes.c_size_t(-1).value
    big = L.taylor_attn_prefill_workspace(4, 16, 4096, 16, 64, 3, TAYLOR_BF16)
    assert big > 0
    assert _prefill(B=4, H=16, N=4096, ws=None, ws_bytes=0) == TAYLOR_ERR_WORKSPACE
    assert _prefill(B=4, H=16, N=4096, ws=FAKE, ws_bytes=big - 1) == TAYLOR_ERR_WORKSPACE
    assert b"workspace" in L.taylor_last_error()


def test_prefill_empty_batch_is_a_no_op():
    # B*H == 0: valid, returns before touching the device
    assert _prefill(B=0, q=None, k=None, v=None, o=None) == TAYLOR_OK
    assert _prefill(H=0, q=None, k=None, v=None, o=None) == TAYLOR_OK


def test_workspace_query():
    assert L.taylor_attn_prefill_workspace(1, 1, 256, 16, 16, 3, TAYLOR_F32) == 0  # one segment
    assert L.taylor_attn_prefill_workspace(1, 1, 256, 16, 16, 2, TAYLOR_F32) == ctypes.c_size_t(-1).value
    # large-width configurations need partial-output space
    w5 = L.taylor_attn_prefill_workspace(2, 8, 8192, 16, 64, 5, TAYLOR_BF16)
    assert w5 >= 8 * 16 * 8192 * 68 * 4
    assert L.taylor_attn_prefill_workspace(0, 8, 8192, 16, 64, 5, TAYLOR_BF16) == 0


def _decode(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=TAYLOR_F32, B=2, H=3, d=16, dv=64, n=3, a=4.0,
                S=FAKE, z=FAKE, o=FAKE, out_dtype=TAYLOR_F32)
    args.update(kw)
    return L.taylor_attn_decode(args["q"], args["k"], args["v"], args["in_dtype"], args["B"],
                                args["H"], args["d"], args["dv"], args["n"], args["a"], args["S"],
                                args["z"], args["o"], args["out_dtype"], None)


def test_decode_rejects_bad_arguments():
    assert _decode(n=4) == TAYLOR_ERR_UNSUPPORTED
    assert _decode(dv=48) == TAYLOR_ERR_UNSUPPORTED
    assert _decode(B=-2) == TAYLOR_ERR_BAD_SHAPE
    assert _decode(a=0.0) == TAYLOR_ERR_BAD_SCALE
    for name in ("q", "k", "v", "S", "z", "o"):
        assert _decode(**{name: None}) == TAYLOR_ERR_NULL_PTR
    assert _decode(B=0, q=None, S=None) == TAYLOR_OK


def test_feature_map_rejects_bad_arguments():
    fm = lambda **kw: L.taylor_feature_map(kw.get("x", FAKE), kw.get("dt", TAYLOR_F32), kw.get("rows", 10),
                                           kw.get("d", 16), kw.get("n", 3), kw.get("a", 4.0),
                                           kw.get("fold", 1), kw.get("phi", FAKE), None)
    assert fm(n=2) == TAYLOR_ERR_UNSUPPORTED
    assert fm(d=17) == TAYLOR_ERR_UNSUPPORTED
    assert fm(rows=-1) == TAYLOR_ERR_BAD_SHAPE
    assert fm(a=-3.0) == TAYLOR_ERR_BAD_SCALE
    assert fm(x=None) == TAYLOR_ERR_NULL_PTR
    assert fm(phi=None) == TAYLOR_ERR_NULL_PTR
    assert fm(rows=0, x=None, phi=None) == TAYLOR_OK


def test_python_wrapper_maps_statuses():
    with pytest.raises(NotImplementedError):
        tl.check(TAYLOR_ERR_UNSUPPORTED)
    with pytest.raises(ValueError):
        tl.check(TAYLOR_ERR_BAD_SHAPE)
    with pytest.raises(RuntimeError):
        tl.check(TAYLOR_ERR_WORKSPACE)


def test_decayed_entry_points_reject_bad_arguments():
    def pre(gamma, **kw):
        args = dict(in_dtype=TAYLOR_BF16, n=3, d=16, ws=None, ws_bytes=0, B=1, H=2, N=64)
        args.update(kw)
        return L.taylor_attn_prefill_decayed(FAKE, FAKE, FAKE, args["in_dtype"], args["B"], args["H"], args["N"],
                                             args["d"], 64,
                                             args["n"], 4.0, gamma, None, None, FAKE, TAYLOR_BF16, None, None,
                                             args["ws"], args["ws_bytes"], None)

    def dec(gamma, **kw):
        return L.taylor_attn_decode_decayed(FAKE, FAKE, FAKE, TAYLOR_F32, 2, 3, 16, 64, kw.get("n", 3), 4.0, gamma,
                                            FAKE, FAKE, FAKE, TAYLOR_F32, None)

    for g in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert pre(g) == TAYLOR_ERR_BAD_SCALE
        assert b"gamma" in L.taylor_last_error()
        assert dec(g) == TAYLOR_ERR_BAD_SCALE
    assert pre(0.9, n=4) == TAYLOR_ERR_UNSUPPORTED
    assert dec(0.9, n=2) == TAYLOR_ERR_UNSUPPORTED
    # the decayed prefill runs the generic kernels: its own workspace size
    need = L.taylor_attn_prefill_decayed_workspace(2, 8, 8192, 16, 64, 3, TAYLOR_BF16)
    assert need != ctypes.c_size_t(-1).value
    assert need > 0
    assert pre(0.9, B=2, H=8, N=8192, ws=FAKE, ws_bytes=need - 1) == TAYLOR_ERR_WORKSPACE
    assert L.taylor_attn_prefill_decayed_workspace(1, 1, 64, 16, 64, 2, TAYLOR_BF16) == ctypes.c_size_t(-1).value


def test_ext_entry_points_reject_bad_arguments():
    def pre(ext):
        return L.taylor_attn_prefill_ext(FAKE, FAKE, FAKE, TAYLOR_BF16, 1, 2, 64, 16, 64, 3, 4.0, ext, None, None,
                                         FAKE, TAYLOR_BF16, None, None, None, 0, None)

    def dec(ext):
        return L.taylor_attn_decode_ext(FAKE, FAKE, FAKE, TAYLOR_F32, 2, 3, 16, 64, 3, 4.0, ext, FAKE, FAKE, FAKE,
                                        TAYLOR_F32, None)

    assert pre(None) == TAYLOR_ERR_NULL_PTR
    assert dec(None) == TAYLOR_ERR_NULL_PTR
    for kw in ({"gamma": 0.0}, {"gamma": 2.0}, {"q_scale": 0.0}, {"k_scale": -1.0}, {"q_scale": float("inf")},
               {"k_scale": float("nan")}):
        opts = dict(gamma=1.0, qk_norm=1, q_scale=1.0, k_scale=1.0, q_head_scale=None)
        opts.update(kw)
        ext = ctypes.byref(tl.Ext(**opts))
        assert pre(ext) == TAYLOR_ERR_BAD_SCALE, kw
        assert dec(ext) == TAYLOR_ERR_BAD_SCALE, kw
    assert (L.taylor_attn_prefill_ext_workspace(2, 8, 8192, 16, 64, 5, TAYLOR_BF16)
            == L.taylor_attn_prefill_decayed_workspace(2, 8, 8192, 16, 64, 5, TAYLOR_BF16))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # the order-4 workload's workspace is larger than the static scratch;
    # the size check comes before any device call
    need = L.taylor_attn_prefill_workspace(2, 8, 8192, 16, 64, 5, TAYLOR_BF16)
    assert need > (128 << 20)
    st = L.taylor_attn_prefill_noalloc(FAKE, FAKE, FAKE, TAYLOR_BF16, 2, 8, 8192, 16, 64, 5, 4.0, None, None,
                                       FAKE, TAYLOR_BF16, None, None, None)
    assert st == TAYLOR_ERR_WORKSPACE
    assert b"scratch" in L.taylor_last_error()
    # argument errors are reported as by taylor_attn_prefill
    st = L.taylor_attn_prefill_noalloc(FAKE, FAKE, FAKE, TAYLOR_BF16, 1, 2, 64, 16, 64, 2, 4.0, None, None,
                                       FAKE, TAYLOR_BF16, None, None, None)
    assert st == TAYLOR_ERR_UNSUPPORTED
