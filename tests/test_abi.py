"""The C-ABI library loads, exports what include/attn.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed: every call here
fails validation, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

from exact_attention_04_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # a non-null, 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(bd.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_error_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert bd.attn_strerror(code) and "unknown" not in bd.attn_strerror(code)
    assert "unknown" in bd.attn_strerror(7)


def fwd_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, Hkv=2, Sq=16, Sk=16, d=128,
             causal=1, scale=0.088, dtype=bd.ATTN_BF16, stream=None)
    a.update(kw)
    return a


def call_fwd(**kw):
    a = fwd_args(**kw)
    return bd.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Sq"], a["Sk"],
                       a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(k=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(v=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(o=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), bd.ATTN_ERR_INVALID_ARG),
    (dict(o=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(Sq=-3), bd.ATTN_ERR_INVALID_ARG),
    (dict(Sk=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(H=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=-0.1), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), bd.ATTN_ERR_INVALID_ARG),
    (dict(d=96), bd.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), bd.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=2), bd.ATTN_ERR_UNSUPPORTED),
    (dict(Sq=1 << 30, H=1 << 20, Hkv=1 << 20), bd.ATTN_ERR_INVALID_ARG),
])
def test_fwd_rejects(kw, code):
    assert call_fwd(**kw) == code


def test_fwd_and_bwd_reject_more_than_2_30_rows():
    assert call_fwd(Sq=(1 << 30) + 1, B=0) == bd.ATTN_ERR_UNSUPPORTED
    assert call_fwd(Sk=(1 << 30) + 1) == bd.ATTN_ERR_UNSUPPORTED
    assert bd.attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, (1 << 30) + 1, 1, 64, 1, 0.1,
                       bd.ATTN_BF16, FAKE, 1 << 40, None) == bd.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(Sq=0), dict(B=0, q=None, o=None, k=None, v=None),
                                dict(Sq=0, q=None, o=None)])
def test_fwd_empty_is_a_noop(kw):
    assert call_fwd(**kw) == bd.ATTN_OK


def verify_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, maxs=3000, stride=3000, o=FAKE, lse=FAKE, B=2, H=32, Hkv=8,
             kq=5, d=128, scale=0.088, dtype=bd.ATTN_BF16, ws=FAKE, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = bd.attn_verify_workspace_bytes(a["B"], a["H"], a["Hkv"], a["kq"], 128)
    return a


def call_verify(**kw):
    a = verify_args(**kw)
    return bd.attn_verify(a["q"], a["k"], a["v"], a["sl"], a["maxs"], a["stride"], a["o"], a["lse"], a["B"],
                          a["H"], a["Hkv"], a["kq"], a["d"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                          a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(k=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(sl=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(sl=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=FAKE + 4), bd.ATTN_ERR_INVALID_ARG),
    (dict(maxs=3001), bd.ATTN_ERR_INVALID_ARG),
    (dict(maxs=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(kq=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(H=30), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.ATTN_ERR_INVALID_ARG),
    (dict(dtype=bd.ATTN_F32), bd.ATTN_ERR_UNSUPPORTED),
    (dict(d=80), bd.ATTN_ERR_UNSUPPORTED),
    (dict(kq=17), bd.ATTN_ERR_UNSUPPORTED),       # 4 heads * 17 tokens > 64 packed rows
    (dict(H=65, Hkv=1, kq=1), bd.ATTN_ERR_UNSUPPORTED),
    (dict(H=8, Hkv=8, kq=65), bd.ATTN_ERR_UNSUPPORTED),
    (dict(wsb=100), bd.ATTN_ERR_WORKSPACE),
])
def test_verify_rejects(kw, code):
    assert call_verify(**kw) == code


def test_verify_workspace_formula():
    # fp32 O and LSE partials for every (sequence, query head, token, piece
    # slot; a (sequence, KV head) segment has at most ceil(256/Hkv) + 2
    # pieces) and one int32 piece count per segment
    up = lambda x: -(-x // 256) * 256
    for B, H, Hkv, kq, d in [(8, 32, 8, 5, 128), (1, 8, 1, 1, 64), (2, 4, 4, 3, 128), (3, 6, 3, 2, 64)]:
        n = B * H * kq * (-(-256 // Hkv) + 2)
        assert bd.attn_verify_workspace_bytes(B, H, Hkv, kq, d) == up(n * d * 4) + up(n * 4) + up(B * Hkv * 4)
    assert bd.attn_verify_workspace_bytes(1, 8, 8, 5, 96) == 0
    assert bd.attn_verify_workspace_bytes(-1, 8, 8, 5, 128) == 0
    assert bd.attn_verify_workspace_bytes(1, 8, 3, 5, 128) == 0


def test_verify_empty_batch_is_a_noop():
    assert call_verify(B=0, q=None, o=None, sl=None, k=None, v=None, ws=None, maxs=0, stride=0) == bd.ATTN_OK


def call_noalloc(**kw):
    a = verify_args(**kw)
    return bd.attn_verify_noalloc(a["q"], a["k"], a["v"], a["sl"], a["maxs"], a["stride"], a["o"], a["lse"], a["B"],
                                  a["H"], a["Hkv"], a["kq"], a["d"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(sl=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(maxs=3001), bd.ATTN_ERR_INVALID_ARG),
    (dict(kq=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(dtype=bd.ATTN_F32), bd.ATTN_ERR_UNSUPPORTED),
    (dict(kq=17), bd.ATTN_ERR_UNSUPPORTED),
    # partials beyond the 32 MiB static scratch (B=12 at the verify workload's
    # other sizes needs 33.7 MB; B=11 fits)
    (dict(B=12), bd.ATTN_ERR_TOO_LARGE),
    (dict(B=64, kq=8), bd.ATTN_ERR_TOO_LARGE),
])
def test_verify_noalloc_rejects(kw, code):
    """Argument checks and the static-scratch limit, all on the host before any HIP call."""
    assert call_noalloc(**kw) == code


def test_verify_noalloc_limit_matches_the_workspace_formula():
    lim = 32 << 20
    assert bd.attn_verify_workspace_bytes(11, 32, 8, 5, 128) <= lim < bd.attn_verify_workspace_bytes(12, 32, 8, 5, 128)
    assert call_noalloc(B=0, q=None, o=None, sl=None, k=None, v=None, maxs=0, stride=0) == bd.ATTN_OK


def paged_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, maxb=100, npages=400, page=64, sl=FAKE, maxs=3000, o=FAKE,
             lse=FAKE, B=2, H=32, Hkv=8, kq=5, d=128, scale=0.088, dtype=bd.ATTN_BF16, ws=FAKE, wsb=None,
             stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = bd.attn_verify_workspace_bytes(a["B"], a["H"], a["Hkv"], a["kq"], 128)
    return a


def call_paged(**kw):
    a = paged_args(**kw)
    return bd.attn_verify_paged(a["q"], a["k"], a["v"], a["table"], a["maxb"], a["npages"], a["page"], a["sl"],
                                a["maxs"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["kq"], a["d"],
                                a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(table=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(page=8), bd.ATTN_ERR_INVALID_ARG),        # below the 16-key half step
    (dict(page=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(page=48), bd.ATTN_ERR_INVALID_ARG),       # not a power of two
    (dict(page=8192), bd.ATTN_ERR_INVALID_ARG),
    (dict(maxs=6401), bd.ATTN_ERR_INVALID_ARG),     # more keys than the table covers (100 * 64)
    (dict(maxb=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(npages=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(k=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(sl=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(H=30), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), bd.ATTN_ERR_INVALID_ARG),
    (dict(dtype=bd.ATTN_F32), bd.ATTN_ERR_UNSUPPORTED),
    (dict(d=96), bd.ATTN_ERR_UNSUPPORTED),
    (dict(kq=17), bd.ATTN_ERR_UNSUPPORTED),
    (dict(H=64, Hkv=1, kq=2), bd.ATTN_ERR_UNSUPPORTED),
    (dict(wsb=100), bd.ATTN_ERR_WORKSPACE),
])
def test_verify_paged_rejects(kw, code):
    assert call_paged(**kw) == code


def test_verify_paged_empty_batch_is_a_noop():
    assert call_paged(B=0, q=None, o=None, sl=None, table=None, k=None, v=None, ws=None, maxs=0,
                      npages=0) == bd.ATTN_OK


def test_verify_tree_rejects_missing_mask():
    a = verify_args()
    args = (a["q"], a["k"], a["v"], a["sl"], a["maxs"], a["stride"])
    tail = (a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["kq"], a["d"], a["scale"], a["dtype"], a["ws"], a["wsb"],
            a["stream"])
    assert bd.attn_verify_tree(*args, None, *tail) == bd.ATTN_ERR_INVALID_ARG
    assert bd.attn_verify_tree(*args, FAKE + 2, *tail) == bd.ATTN_ERR_INVALID_ARG
    # 32-bit masks: at most 32 tree nodes, even where 64 packed rows would fit
    a = verify_args(H=8, Hkv=8, kq=33)
    tail = (a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["kq"], a["d"], a["scale"], a["dtype"], a["ws"], a["wsb"],
            a["stream"])
    assert bd.attn_verify_tree(*args, FAKE, *tail) == bd.ATTN_ERR_UNSUPPORTED
    a = verify_args(H=8, Hkv=4, kq=33)  # 66 packed rows
    tail = (a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["kq"], a["d"], a["scale"], a["dtype"], a["ws"], a["wsb"],
            a["stream"])
    assert bd.attn_verify_tree(*args, FAKE, *tail) == bd.ATTN_ERR_UNSUPPORTED
    a0 = verify_args(B=0, q=None, o=None, sl=None, k=None, v=None, ws=None, maxs=0, stride=0)
    assert bd.attn_verify_tree(a0["q"], a0["k"], a0["v"], a0["sl"], 0, 0, None, a0["o"], a0["lse"], 0, a0["H"],
                               a0["Hkv"], a0["kq"], a0["d"], a0["scale"], a0["dtype"], None, a0["wsb"],
                               None) == bd.ATTN_OK


def call_spec(**kw):
    a = dict(x=FAKE, q=FAKE, p=FAKE, ua=FAKE, us=FAKE, n=FAKE, out=FAKE, B=8, k=5, V=32000, ws=FAKE, wsb=None,
             stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = bd.attn_spec_accept_workspace_bytes(a["B"], a["V"])
    return bd.attn_spec_accept(a["x"], a["q"], a["p"], a["ua"], a["us"], a["n"], a["out"], a["B"], a["k"], a["V"],
                               a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(p=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ua=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(us=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(n=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(out=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=FAKE + 4), bd.ATTN_ERR_INVALID_ARG),
    (dict(k=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(V=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(V=(1 << 22) + 1), bd.ATTN_ERR_UNSUPPORTED),
    (dict(wsb=8), bd.ATTN_ERR_WORKSPACE),
])
def test_spec_accept_rejects(kw, code):
    assert call_spec(**kw) == code


def test_spec_accept_workspace_and_noop():
    # two int64 sums per (sequence, 4096-entry chunk), 16-byte aligned, then one int32 per sequence
    assert bd.attn_spec_accept_workspace_bytes(8, 4096) == 8 * 1 * 16 + 8 * 4
    assert bd.attn_spec_accept_workspace_bytes(8, 4097) == 8 * 2 * 16 + 8 * 4
    assert bd.attn_spec_accept_workspace_bytes(3, 4096) == 48 + 3 * 4
    assert bd.attn_spec_accept_workspace_bytes(1, 0) == 0
    assert bd.attn_spec_accept_workspace_bytes(1, (1 << 22) + 1) == 0
    assert call_spec(B=0, x=None, q=None, p=None, ua=None, us=None, n=None, out=None, ws=None) == bd.ATTN_OK
    # k = 0 needs no draft arrays
    assert call_spec(k=0, x=None, q=None, ua=None, wsb=0) == bd.ATTN_ERR_WORKSPACE


def call_bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=4, Hkv=2, Sq=16,
             Sk=16, d=128, causal=1, scale=0.088, dtype=bd.ATTN_BF16, ws=FAKE, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = bd.attn_bwd_workspace_bytes(a["B"], a["H"], a["Sq"])
    return bd.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["H"],
                       a["Hkv"], a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                       a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(k=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(v=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(o=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(do=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(lse=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), bd.ATTN_ERR_INVALID_ARG),
    (dict(dq=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(dk=FAKE + 8), bd.ATTN_ERR_INVALID_ARG),
    (dict(dv=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), bd.ATTN_ERR_INVALID_ARG),
    (dict(ws=FAKE + 4), bd.ATTN_ERR_INVALID_ARG),
    (dict(wsb=16), bd.ATTN_ERR_WORKSPACE),
    (dict(H=3), bd.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), bd.ATTN_ERR_INVALID_ARG),
    (dict(Sq=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(Sk=-1), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), bd.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.ATTN_ERR_INVALID_ARG),
    (dict(d=96), bd.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=bd.ATTN_F32), bd.ATTN_ERR_UNSUPPORTED),
])
def test_bwd_rejects(kw, code):
    assert call_bwd(**kw) == code


def test_bwd_workspace_and_noop():
    # two 256-byte aligned fp32 arrays of B*H*Sq
    assert bd.attn_bwd_workspace_bytes(1, 4, 16) == 2 * 256
    assert bd.attn_bwd_workspace_bytes(2, 32, 8192) == 2 * 2 * 32 * 8192 * 4
    assert bd.attn_bwd_workspace_bytes(1, 1, 65) == 2 * 512
    assert bd.attn_bwd_workspace_bytes(0, 4, 16) == 0
    assert bd.attn_bwd_workspace_bytes(-1, 4, 16) == 0
    nothing = dict(q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, ws=None)
    assert call_bwd(B=0, **nothing) == bd.ATTN_OK
    assert call_bwd(Sq=0, Sk=0, **nothing) == bd.ATTN_OK


def test_package_exports_every_binding_entry_point():
    import exact_attention_04_amd as pkg
    for name in bd.EXPORTED + ("fwd", "bwd", "verify", "verify_tree", "verify_paged", "spec_accept"):
        assert name in pkg.__all__, name
        assert getattr(pkg, name) is getattr(bd, name)
