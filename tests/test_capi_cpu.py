"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and its host-side argument checks return the documented
status codes before anything is enqueued (no call here reaches the device).
"""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_sigmoid_amd as moe
from mixture_experts_layer_sigmoid_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

OK, INVALID, UNSUPPORTED, ALIGN, WS = 0, -1, -2, -3, -4
A = 0x10000  # aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run __graft_entry__.build())")
    return L.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 1
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(-4) == b"workspace missing or too small"


def _route(lib, **kw):
    a = dict(x=A, x_fmt=1, w=A, bias=A, lin=None, T=4, H=64, E=16, ng=4, tg=2, k=4, scale=1.0,
             lout=None, idx=A, w_out=A)
    a.update(kw)
    return lib.moe_route(a["x"], a["x_fmt"], a["w"], a["bias"], a["lin"], a["T"], a["H"], a["E"],
                         a["ng"], a["tg"], a["k"], a["scale"], a["lout"], a["idx"], a["w_out"],
                         a.get("ws"), a.get("wsb", 0), None)


def test_route_validation(lib):
    assert _route(lib, E=0) == INVALID
    assert _route(lib, E=513) == INVALID
    assert _route(lib, ng=3) == INVALID                 # 16 % 3
    assert _route(lib, E=8, ng=8, tg=2, k=2) == INVALID  # groups of 1
    assert _route(lib, tg=5) == INVALID
    assert _route(lib, k=9) == INVALID                  # > topk_group * E / n_group
    assert _route(lib, k=17, E=64, ng=1, tg=1) == INVALID
    assert _route(lib, bias=None) == INVALID
    assert _route(lib, x_fmt=2) == UNSUPPORTED
    assert _route(lib, H=48) == INVALID                 # bf16 needs H % 32
    assert _route(lib, x=A + 8) == ALIGN
    assert b"aligned" in lib.moe_last_error()
    assert _route(lib, T=0) == OK                       # nothing to do, nothing launched
    assert _route(lib, T=0, x=None, w=None, lin=A) == OK
    assert _route(lib) == WS                            # the GEMM needs its workspace
    need = lib.moe_route_workspace(4, 64, 16)
    assert need >= 4 * 16 * 4
    assert _route(lib, ws=A, wsb=need - 1) == WS
    assert lib.moe_route_workspace(0, 64, 16) == 0


def test_route_empty_batch_takes_null_pointers(lib):
    assert lib.moe_route(None, 1, None, None, None, 0, 256, 8, 2, 1, 2, 1.0, None, None, None,
                         None, 0, None) == OK
    assert lib.moe_route(None, 1, None, None, None, 0, 256, 8, 3, 1, 2, 1.0, None, None, None,
                         None, 0, None) == INVALID      # limits are still checked


def test_grouped_fc_empty_calls_take_null_pointers(lib):
    for f in (1, 2):
        assert lib.moe_grouped_fc1_swiglu(None, None, f, None, None, None, f, None, 8, 256, 128, 0,
                                          None, None, None, None) == OK
        assert lib.moe_grouped_fc2(None, None, f, None, None, f, None, 8, 256, 128, 0, None, 1,
                                   None) == OK
    assert lib.moe_grouped_fc2(None, None, 2, None, None, 2, None, 8, 250, 128, 0, None, 1,
                               None) == INVALID         # shapes are still checked


def test_quantize_validation(lib):
    q = lambda **k: lib.moe_quantize_mx(k.get("inp", A), k.get("fi", 1), k.get("rows", 4),
                                        k.get("K", 64), k.get("axis", 0), k.get("fo", 2),
                                        k.get("c", A), k.get("s", A), None)
    assert q(K=48) == INVALID
    assert q(axis=2) == INVALID
    assert q(axis=1, fi=0) == UNSUPPORTED       # axis 1 takes bf16 only
    assert q(axis=1, rows=40) == INVALID        # axis 1 needs rows % 32 == 0
    assert q(fo=1) == UNSUPPORTED
    assert q(fi=2) == UNSUPPORTED
    assert q(c=A + 4) == ALIGN
    assert q(rows=0) == OK


def test_permute_bounds_and_validation(lib):
    assert lib.moe_permute_rows_bound(64, 4, 16, 32) == 64 * 4 + 16 * 31
    assert lib.moe_permute_rows_bound(-1, 4, 16, 1) == -1
    ws = lib.moe_permute_workspace(4096, 8, 256)
    assert ws == 32 * 256 * 4
    p = lambda **k: lib.moe_permute(A, k.get("T", 8), 2, 4, k.get("align", 1), k.get("rin"),
                                    k.get("rb", 0), None, 0, A, A, A, A, k.get("rout"), None,
                                    k.get("ws", A), k.get("wsb", 1 << 20), None)
    assert p(align=3) == INVALID
    assert p(wsb=0) == WS
    assert p(ws=None) == WS
    assert p(rin=A) == INVALID                  # rows_in without rows_out
    assert p(rin=A, rout=A, rb=24) == ALIGN
    assert p(T=-1) == INVALID


def test_grouped_mlp_validation(lib):
    need = lib.moe_grouped_mlp_workspace(8, 256, 128, 100, 1, 1)
    assert need >= 100 * 128 * 2

    def g(**k):
        return lib.moe_grouped_mlp_fwd(A, k.get("asc"), k.get("af", 1), None, A, k.get("w1s"), A,
                                       k.get("w2s"), k.get("wf", 1), A, 8, k.get("H", 256),
                                       k.get("F", 128), 100, None, k.get("y", A), k.get("yf", 1),
                                       k.get("ws", A), k.get("wsb", need), None)
    assert g(wf=0) == UNSUPPORTED
    assert g(af=2, wf=2, yf=1) == INVALID or g(af=2, wf=2, yf=1) == UNSUPPORTED
    assert g(H=200) == INVALID
    assert g(F=96) == INVALID
    assert g(y=A + 2) == ALIGN
    assert g(wsb=need - 1) == WS
    assert g(af=3, wf=3, yf=1, H=256, F=128, asc=A, w1s=A, w2s=A) == INVALID   # fp4 needs F % 256


def test_shared_fold_validation(lib):
    """fc1 / fc2 with the shared expert folded in: the extra weights are
    required, fp32 layers are refused, and an empty call is a no-op."""
    def f1(**k):
        return lib.moe_grouped_fc1_swiglu_dense(
            A, k.get("asc", A), k.get("af", 1), A, A, A, k.get("af", 1), A, 8, 256, 128,
            k.get("rows", 100), None, A, A, k.get("w1d", A), k.get("w1ds", A), k.get("T", 20), None)

    def f2(**k):
        return lib.moe_grouped_fc2_dense(
            A, k.get("hsc", A), k.get("hf", 2), A, A, k.get("hf", 2), A, 8, 256, 128,
            k.get("rows", 100), k.get("y", A), 1, k.get("w2d", A), k.get("w2ds", A),
            k.get("T", 20), None)
    assert f1(af=0) == UNSUPPORTED
    assert f2(hf=0) == UNSUPPORTED
    assert f1(w1d=None) == INVALID
    assert f2(w2d=None) == INVALID
    assert f2(w2ds=None) == INVALID               # MX weights need their scales
    assert f1(af=2, w1ds=A + 2) == ALIGN
    assert f2(y=A + 8) == ALIGN
    assert f1(T=-1) == INVALID
    assert f1(rows=0, T=0) == OK
    assert f2(rows=0, T=0) == OK


def test_combine_validation(lib):
    c = lambda **k: lib.moe_combine(A, k.get("yf", 1), A, A, None, k.get("T", 4), k.get("k", 2),
                                    k.get("H", 64), k.get("out", A), k.get("of", 1), None)
    assert c(H=60) == INVALID
    assert c(k=17) == INVALID
    assert c(yf=2) == UNSUPPORTED
    assert c(out=A + 4) == ALIGN
    assert c(T=0) == OK


def test_binding_raises_with_message(lib):
    with pytest.raises(moe.MoEError) as ei:
        L._check("moe_route", _route(lib, E=0))
    assert "E must be" in str(ei.value)


def test_backward_validation(lib):
    assert lib.moe_segments_kstride(1000, 8) == ((1000 + 8 * 127 + 127) // 128) * 128
    assert lib.moe_segments_kstride(-1, 8) == -1
    assert lib.moe_segments_kstride(0, 0) == -1
    # combine backward: bad k, unsupported dout format, alignment
    cb = lambda **k: lib.moe_combine_bwd(k.get("d", A), k.get("df", 1), A, A, A, 4, k.get("k", 2),
                                         k.get("H", 64), 32, k.get("dy", A), k.get("of", 1),
                                         k.get("ds", A), None, None)
    assert cb(k=0) == INVALID
    assert cb(df=2) == UNSUPPORTED
    assert cb(of=7) == UNSUPPORTED
    assert cb(of=2, H=72) == INVALID              # MX dy needs H % 32 == 0
    assert cb(of=2, ds=None) == INVALID           # MX dy needs its scales
    assert cb(dy=A + 2) == ALIGN
    un = lambda **k: lib.moe_unpermute(A, k.get("f", 1), A, 4, k.get("k", 2), k.get("H", 64), A,
                                       k.get("of", 1), None)
    assert un(H=60) == INVALID
    assert un(k=0) == INVALID
    assert un(k=17) == INVALID                    # the summing kernel holds at most 16 slots
    assert un(of=3) == UNSUPPORTED
    qs = lambda **k: lib.moe_quantize_mx_segments(
        A, k.get("fi", 1), k.get("mode", 0), k.get("src", A), A, None, 4, k.get("rows", 128),
        k.get("C", 64), k.get("ks", 1024), k.get("fo", 2), A, A, A, None)
    assert qs(mode=3) == INVALID
    assert qs(fo=1) == UNSUPPORTED
    assert qs(fo=3) == UNSUPPORTED                # stage-major segments are E4M3 only
    assert qs(C=60) == INVALID
    assert qs(fi=2) == UNSUPPORTED
    assert qs(ks=256) == INVALID                  # below moe_segments_kstride(128, 4)
    assert qs(src=None) == INVALID
    # grouped GEMMs: bad shapes and formats are rejected before any launch
    d2 = lambda **k: lib.moe_grouped_fc2_dgrad_dswiglu(
        A, A, k.get("f", 2), A, A, A, 4, k.get("H", 256), k.get("F", 128), 64, A, A, A, None, None)
    assert d2(H=200) == INVALID
    assert d2(f=0) == UNSUPPORTED
    d1 = lambda **k: lib.moe_grouped_fc1_dgrad(A, A, k.get("f", 2), A, A, A, 4, k.get("H", 256),
                                               k.get("F", 128), 64, A, None)
    assert d1(F=100) == INVALID
    wg = lambda **k: lib.moe_grouped_wgrad(A, A, A, A, k.get("f", 2), A, 4, k.get("M", 256),
                                           k.get("N", 256), k.get("ks", 1024), A, None)
    assert wg(f=3) == UNSUPPORTED
    assert wg(M=96) == INVALID
    assert wg(ks=1000) == INVALID


def test_shared_fold_selection_and_buffers(lib):
    """Host logic of MoEForward: the shared expert is folded into the routed
    launches exactly when its width equals the routed experts', the layer is
    not fp32 and the batch is not empty; folded, its rows follow the routed
    rows in h and y (y_shared is a view of them)."""
    kw = dict(H=256, F=128, E=8, n_group=2, topk_group=1, k=2, routed_scale=1.0, device="cpu")
    fw = moe.MoEForward(T=4, fmt="bf16", F_shared=128, **kw)
    assert fw.fuse_shared
    assert fw.y_rows.shape == (fw.bound + 4, 256) and fw.h.shape == (fw.bound + 4, 128)
    assert fw.y_shared.data_ptr() == fw.y_rows[fw.bound].data_ptr()
    assert not moe.MoEForward(T=4, fmt="fp32", F_shared=128, **kw).fuse_shared
    assert not moe.MoEForward(T=4, fmt="bf16", F_shared=256, **kw).fuse_shared
    assert not moe.MoEForward(T=0, fmt="bf16", F_shared=128, **kw).fuse_shared
    assert not moe.MoEForward(T=4, fmt="bf16", F_shared=128, fuse_shared=False, **kw).fuse_shared
    with pytest.raises(ValueError):
        moe.MoEForward(T=4, fmt="bf16", F_shared=256, fuse_shared=True, **kw)
    with pytest.raises(RuntimeError):
        fw.shared(None, None)


def test_grouped_mlp_bwd_validation(lib):
    """moe_grouped_mlp_bwd checks everything before its first kernel."""
    T, k, E, H, F, rows = 64, 6, 48, 512, 384, 64 * 6 + 48 * 31
    need = lib.moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, 2)
    assert need > 0
    assert lib.moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, 1) == 0    # MXFP8 only
    assert lib.moe_grouped_mlp_bwd_workspace(T, k, E, 500, F, rows, 2) == 0  # H % 128
    assert lib.moe_grouped_mlp_bwd_workspace(T, k, E, H, F, T * k - 1, 2) == 0

    def call(**kw):
        a = dict(dout=A, x=A, af=1, rm=A, src=A, tw=A, off=A, save=A, w1t=A, w1s=A, w2t=A, w2s=A,
                 f=2, T=T, k=k, E=E, H=H, F=F, rows=rows, dx=A, dw1=A, dw2=A, ws=A, wsb=need)
        a.update(kw)
        return lib.moe_grouped_mlp_bwd(a["dout"], a["x"], a["af"], a["rm"], a["src"], a["tw"],
                                       a["off"], a["save"], a["w1t"], a["w1s"], a["w2t"], a["w2s"],
                                       a["f"], a["T"], a["k"], a["E"], a["H"], a["F"], a["rows"],
                                       a["dx"], a["dw1"], a["dw2"], a["ws"], a["wsb"], None)
    assert call(f=3) == UNSUPPORTED
    assert call(af=2) == UNSUPPORTED
    assert call(k=17) == INVALID
    assert call(F=200) == INVALID
    assert call(E=1025) == INVALID
    assert call(rows=T * k - 1) == INVALID
    assert call(src=None) == INVALID
    assert call(dout=None) == INVALID
    assert call(dw1=A + 8) == ALIGN
    assert call(w1s=A + 2) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert b"moe_grouped_mlp_bwd_workspace" in lib.moe_last_error()


def test_route_bwd_validation(lib):
    T, k, E, H = 300, 8, 32, 512
    need = lib.moe_route_bwd_workspace(T, H, E, 100)
    assert need > 0 and lib.moe_route_bwd_workspace(T, H, E, 7) == 0    # 7 does not divide 300

    def call(**kw):
        a = dict(dout=A, y=A, af=1, rm=A, idx=A, lg=A, x=A, wr=A, T=T, k=k, E=E, H=H, sc=2.5, L=100,
                 al=0.01, dl=None, loss=A, dx=A, dw=A, ws=A, wsb=need)
        a.update(kw)
        return lib.moe_route_bwd(a["dout"], a["y"], a["af"], a["rm"], a["idx"], a["lg"], a["x"],
                                 a["wr"], a["T"], a["k"], a["E"], a["H"], a["sc"], a["L"], a["al"],
                                 a["dl"], a["loss"], a["dx"], a["dw"], a["ws"], a["wsb"], None)
    assert call(af=0) == UNSUPPORTED
    assert call(E=36) == INVALID                 # E % 8
    assert call(k=17) == INVALID
    assert call(L=7) == INVALID
    assert call(loss=None) == INVALID            # the balance loss needs its output
    assert call(x=A + 4) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(T=0, dout=None, y=None) == OK    # empty batch: nothing to do
    assert lib.moe_bias_update(A, 0, 1e-3, A, A, None) == INVALID
    assert lib.moe_bias_update(None, 8, 1e-3, A, A, None) == INVALID


def test_nvfp4_validation(lib):
    """NVFP4 quantizer, tensor scale, pack and the W4A4 fc1 / fc2 entries."""
    q = lambda **k: lib.moe_quantize_nvfp4(k.get("inp", A), k.get("fi", 1), k.get("rows", 4),
                                           k.get("K", 64), k.get("rpt", 4), k.get("g", A),
                                           k.get("c", A), k.get("s", A), k.get("v"), None)
    assert q(K=40) == INVALID                    # blocks of 16
    assert q(rpt=0) == INVALID
    assert q(fi=2) == UNSUPPORTED
    assert q(c=None, s=None) == INVALID          # no output
    assert q(c=A + 4) == ALIGN
    assert q(v=A + 8) == ALIGN
    assert q(g=None) == INVALID
    assert q(rows=0, inp=None, g=None) == OK
    ts = lambda **k: lib.moe_nvfp4_tensor_scale(k.get("inp", A), k.get("fi", 1), k.get("n", 2),
                                                k.get("per", 64), k.get("g", A), None)
    assert ts(n=0) == INVALID
    assert ts(per=0) == INVALID
    assert ts(fi=3) == UNSUPPORTED
    assert ts(g=None) == INVALID
    pk = lambda **k: lib.moe_pack_weights(A, k.get("sc", A), 4, 2, k.get("N", 128), k.get("K", 128),
                                          k.get("half", 64), A, k.get("osc", A), None)
    assert pk(K=96) == INVALID                   # 64-value stages
    assert pk(N=96, half=48) == INVALID
    assert pk(sc=None) == INVALID
    assert pk(osc=A + 2) == ALIGN
    f1 = lambda **k: lib.moe_grouped_fc1_swiglu_nvfp4(
        k.get("a", A), None, A, k.get("ws", A), A, k.get("xg", 2.0 ** -8), 2.0 ** -6, A, 8,
        k.get("H", 256), k.get("F", 128), k.get("rows", 100), k.get("h", A), None)
    assert f1(H=192) == INVALID
    assert f1(F=96) == INVALID
    assert f1(xg=0.0) == INVALID
    assert f1(h=A + 8) == ALIGN
    assert f1(ws=A + 1) == ALIGN
    assert f1(rows=0, a=None, h=None) == OK
    f2 = lambda **k: lib.moe_grouped_fc2_nvfp4(A, A, A, A, k.get("hg", 2.0 ** -6), A, k.get("E", 8),
                                               256, 128, 100, k.get("y", A), None)
    assert f2(E=0) == INVALID
    assert f2(hg=-1.0) == INVALID
    assert f2(y=A + 2) == ALIGN
    # the generic grouped entries do not take NVFP4 (its tensor scales are
    # arguments of the NVFP4 entries only)
    assert lib.moe_grouped_fc2(A, A, 4, A, A, 4, A, 8, 256, 128, 100, A, 1, None) == UNSUPPORTED
    assert lib.moe_quantize_mx(A, 1, 4, 64, 0, 4, A, A, None) == UNSUPPORTED
