"""C ABI of libteaf.so on the CPU: the library loads, exports every declared entry point, and
rejects invalid arguments with the documented status before touching the GPU.

No test here passes arguments that would reach a kernel launch.
"""
import ctypes
import os
import re

import pytest

import tiled_exact_attention_forward_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# A fake, 16-byte aligned, non-null "device pointer". Every call below is rejected by the
# host-side checks before it could be used.
P = ctypes.c_void_p(0x1000)
N = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert fa.fa_status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5, -6):
        assert fa.fa_status_string(s) and fa.fa_status_string(s) != "unknown status"
    assert fa.fa_status_string(42) == "unknown status"
    assert fa.fa_version() >= 10000


def fwd(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nkv=8, d=64, scale=0.125, mask=0, W=0, G=0,
        dtype=1):
    return fa.load_library().fa_forward(q, k, v, o, lse, B, H, Nq, Nkv, d, scale, mask, W, G,
                                        dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=N), fa.FA_ERR_NULL), (dict(k=N), fa.FA_ERR_NULL), (dict(v=N), fa.FA_ERR_NULL),
    (dict(o=N), fa.FA_ERR_NULL), (dict(lse=N), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE), (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(Nkv=-3), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED), (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=5), fa.FA_ERR_UNSUPPORTED), (dict(mask=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=3, W=-1), fa.FA_ERR_SHAPE), (dict(mask=4, G=-1), fa.FA_ERR_SHAPE),
    (dict(mask=2, W=0, G=0), fa.FA_ERR_SHAPE), (dict(mask=2, W=4, G=-1), fa.FA_ERR_SHAPE),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE),
    (dict(q=ctypes.c_void_p(0x1008)), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 16), fa.FA_ERR_SHAPE),
    # 2^24 workgroups of 256 threads: one work-item past a dispatch's 32-bit grid
    (dict(B=1 << 16, H=256, Nq=128, Nkv=128), fa.FA_ERR_SHAPE),
])
def test_forward_rejects_before_launch(kw, status):
    assert fwd(**kw) == status


def dec(q=P, kp=P, vp=P, pt=P, sl=P, o=P, lse=N, page=256, S=8, H=32, d=128, maxp=32, npages=300,
        scale=0.088, dtype=1, ws=P, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.fa_decode_paged_workspace_bytes(S, H, d, maxp, page)
    return lib.fa_decode_paged(q, kp, vp, pt, sl, o, lse, page, S, H, d, maxp, npages, scale,
                               dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=N), fa.FA_ERR_NULL), (dict(kp=N), fa.FA_ERR_NULL), (dict(vp=N), fa.FA_ERR_NULL),
    (dict(pt=N), fa.FA_ERR_NULL), (dict(sl=N), fa.FA_ERR_NULL), (dict(o=N), fa.FA_ERR_NULL),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE), (dict(maxp=0), fa.FA_ERR_SHAPE),
    (dict(npages=0), fa.FA_ERR_SHAPE),
    (dict(page=128), fa.FA_ERR_UNSUPPORTED), (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED), (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(H=12), fa.FA_ERR_UNSUPPORTED),
    # launch-grid dimensions: splits (one per page when there are many), sequences, heads
    (dict(maxp=65536), fa.FA_ERR_SHAPE), (dict(S=65536), fa.FA_ERR_SHAPE),
    (dict(H=65536), fa.FA_ERR_SHAPE),
    (dict(ws=N), fa.FA_ERR_WORKSPACE), (dict(wsb=16), fa.FA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1004)), fa.FA_ERR_WORKSPACE),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE),
])
def test_decode_rejects_before_launch(kw, status):
    assert dec(**kw) == status


def dec_noalloc(q=P, kp=P, vp=P, pt=P, sl=P, o=P, lse=N, page=256, S=8, H=32, d=128, maxp=32,
                npages=300, scale=0.088, dtype=1):
    return fa.load_library().fa_decode_paged_noalloc(q, kp, vp, pt, sl, o, lse, page, S, H, d,
                                                     maxp, npages, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=N), fa.FA_ERR_NULL), (dict(pt=N), fa.FA_ERR_NULL), (dict(o=N), fa.FA_ERR_NULL),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(maxp=0), fa.FA_ERR_SHAPE),
    (dict(page=128), fa.FA_ERR_UNSUPPORTED), (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED), (dict(H=12), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE), (dict(maxp=65536), fa.FA_ERR_SHAPE),
    # partials beyond the 16 MiB static array, even at the longest split (256 tokens), which
    # these sizes pick: 64 x 64 x 64 pages take 135 MB, 32 x 32 x 64 pages 33.8 MB
    (dict(S=64, H=64, maxp=64), fa.FA_ERR_SCRATCH),
    (dict(S=32, H=32, maxp=64), fa.FA_ERR_SCRATCH),
])
def test_decode_noalloc_rejects_before_launch(kw, status):
    assert dec_noalloc(**kw) == status


def bs(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nkv=8, d=64, scale=0.125, layout=P,
       block=128, dtype=1):
    return fa.load_library().fa_forward_block_sparse(q, k, v, o, lse, B, H, Nq, Nkv, d, scale,
                                                     layout, block, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=None), fa.FA_ERR_NULL), (dict(q=None), fa.FA_ERR_NULL),
    (dict(block=64), fa.FA_ERR_UNSUPPORTED), (dict(block=256), fa.FA_ERR_UNSUPPORTED),
    (dict(Nkv=262145), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED), (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE),
])
def test_block_sparse_rejects_before_launch(kw, status):
    assert bs(**kw) == status


def test_decode_workspace_bytes():
    lib = fa.load_library()
    # 8 sequences, 32 heads, d 128, 32 pages of 256 tokens: 128 splits of 64 tokens,
    # each split keeps 128 partial outputs and one log-sum-exp (float32)
    assert lib.fa_decode_paged_workspace_bytes(8, 32, 128, 32, 256) == 8 * 32 * 128 * 129 * 4
    assert lib.fa_decode_paged_workspace_bytes(0, 32, 128, 32, 256) == 0


def bwd(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, Nq=8, Nkv=8, d=64,
        scale=0.125, mask=0, W=0, G=0, dtype=1, ws=P, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.fa_backward_workspace_bytes(B, H, Nq)
    return lib.fa_backward(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nkv, d, scale, mask, W, G,
                           dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=N), fa.FA_ERR_NULL), (dict(o=N), fa.FA_ERR_NULL), (dict(lse=N), fa.FA_ERR_NULL),
    (dict(do=N), fa.FA_ERR_NULL), (dict(dq=N), fa.FA_ERR_NULL), (dict(dk=N), fa.FA_ERR_NULL),
    (dict(dv=N), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(Nkv=0), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED), (dict(mask=5), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=2, W=0), fa.FA_ERR_SHAPE), (dict(mask=3, W=-2), fa.FA_ERR_SHAPE),
    (dict(mask=4, G=-1), fa.FA_ERR_SHAPE), (dict(scale=float("nan")), fa.FA_ERR_SHAPE),
    (dict(ws=N), fa.FA_ERR_WORKSPACE), (dict(wsb=8 * 4), fa.FA_ERR_WORKSPACE),
    (dict(dk=ctypes.c_void_p(0x1002)), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 16, wsb=1 << 62), fa.FA_ERR_SHAPE),
])
def test_backward_rejects_before_launch(kw, status):
    assert bwd(**kw) == status


def bwd_bs(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, Nq=8, Nkv=8, d=64,
           scale=0.125, layout=P, block=128, dtype=1, ws=P, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.fa_backward_workspace_bytes(B, H, Nq)
    return lib.fa_backward_block_sparse(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nkv, d, scale,
                                        layout, block, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=N), fa.FA_ERR_NULL), (dict(q=N), fa.FA_ERR_NULL), (dict(dv=N), fa.FA_ERR_NULL),
    (dict(block=64), fa.FA_ERR_UNSUPPORTED), (dict(Nkv=262145), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=262145), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED), (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE), (dict(ws=N), fa.FA_ERR_WORKSPACE),
    (dict(wsb=8 * 4), fa.FA_ERR_WORKSPACE), (dict(dq=ctypes.c_void_p(0x1004)), fa.FA_ERR_UNSUPPORTED),
])
def test_backward_block_sparse_rejects_before_launch(kw, status):
    assert bwd_bs(**kw) == status


def test_backward_workspace_bytes():
    lib = fa.load_library()
    # per 32-row tile of each (b, h): 32 log2-scaled LSE values and 32 values of D (floats)
    assert lib.fa_backward_workspace_bytes(2, 3, 100) == 2 * 3 * 4 * 64 * 4
    assert lib.fa_backward_workspace_bytes(1, 1, 0) == 0


def pre(q=P, kp=P, vp=P, pt=P, sl=P, ql=P, o=P, lse=P, page=256, S=4, Qm=64, H=8, d=128,
        maxp=8, npages=40, scale=0.088, mask=1, W=0, G=0, dtype=2):
    return fa.load_library().fa_prefill_paged(q, kp, vp, pt, sl, ql, o, lse, page, S, Qm, H, d,
                                              maxp, npages, scale, mask, W, G, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=N), fa.FA_ERR_NULL), (dict(kp=N), fa.FA_ERR_NULL), (dict(pt=N), fa.FA_ERR_NULL),
    (dict(sl=N), fa.FA_ERR_NULL), (dict(ql=N), fa.FA_ERR_NULL), (dict(o=N), fa.FA_ERR_NULL),
    (dict(lse=N), fa.FA_ERR_NULL),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(Qm=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE),
    (dict(maxp=0), fa.FA_ERR_SHAPE), (dict(npages=0), fa.FA_ERR_SHAPE),
    (dict(page=128), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED), (dict(mask=5), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=2, W=0), fa.FA_ERR_SHAPE), (dict(mask=3, W=-1), fa.FA_ERR_SHAPE),
    (dict(mask=4, G=-1), fa.FA_ERR_SHAPE), (dict(H=70000), fa.FA_ERR_SHAPE),
    (dict(maxp=1 << 23), fa.FA_ERR_SHAPE), (dict(scale=float("nan")), fa.FA_ERR_SHAPE),
    (dict(o=ctypes.c_void_p(0x1008)), fa.FA_ERR_UNSUPPORTED),
])
def test_prefill_paged_rejects_before_launch(kw, status):
    assert pre(**kw) == status


def mrg(oa=P, la=P, ob=P, lb=P, o=P, l=P, rows=10, d=128, dtype=2):
    return fa.load_library().fa_merge_lse(oa, la, ob, lb, o, l, rows, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(oa=N), fa.FA_ERR_NULL), (dict(lb=N), fa.FA_ERR_NULL), (dict(o=N), fa.FA_ERR_NULL),
    (dict(l=N), fa.FA_ERR_NULL), (dict(rows=0), fa.FA_ERR_SHAPE),
    (dict(rows=1 << 41), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(rows=1 << 28), fa.FA_ERR_SHAPE),  # bf16 d 128: 16 threads a row, 2^24 workgroups
    (dict(dtype=4), fa.FA_ERR_UNSUPPORTED), (dict(ob=ctypes.c_void_p(0x1004)),
                                             fa.FA_ERR_UNSUPPORTED),
])
def test_merge_rejects_before_launch(kw, status):
    assert mrg(**kw) == status


def mm(qi=P, ki=P, vi=P, qt=P, kt=P, vt=P, oi=P, li=P, ot=P, lt=P, B=1, H=2, ni=9, nt=14, d=64,
       scale=0.1, dtype=2, mode=0, ws=P, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.fa_multimodal_workspace_bytes(B, H, nt, d, dtype)
    return lib.fa_multimodal_forward(qi, ki, vi, qt, kt, vt, oi, li, ot, lt, B, H, ni, nt, d,
                                     scale, dtype, mode, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qi=N), fa.FA_ERR_NULL), (dict(vt=N), fa.FA_ERR_NULL), (dict(lt=N), fa.FA_ERR_NULL),
    (dict(oi=N), fa.FA_ERR_NULL), (dict(ni=0), fa.FA_ERR_SHAPE), (dict(nt=0), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED), (dict(dtype=9), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=N), fa.FA_ERR_WORKSPACE), (dict(wsb=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1001)), fa.FA_ERR_WORKSPACE),
    (dict(scale=float("nan")), fa.FA_ERR_SHAPE), (dict(mode=2), fa.FA_ERR_UNSUPPORTED),
    (dict(mode=1, ni=33), fa.FA_ERR_UNSUPPORTED), (dict(mode=1, ni=64, dtype=0),
                                                   fa.FA_ERR_UNSUPPORTED),
])
def test_multimodal_rejects_before_launch(kw, status):
    assert mm(**kw) == status


def test_multimodal_workspace_bytes():
    lib = fa.load_library()
    rows = 2 * 3 * 100
    # the text-to-image partial output (rounded up to 256 bytes) and its row LSE
    assert lib.fa_multimodal_workspace_bytes(2, 3, 100, 128, 2) == \
        ((rows * 128 * 2 + 255) // 256) * 256 + rows * 4
    assert lib.fa_multimodal_workspace_bytes(2, 3, 100, 64, 0) == \
        ((rows * 64 * 4 + 255) // 256) * 256 + rows * 4
