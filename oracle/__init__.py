"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the benchmark's CPU-baseline leg may import
this package. It is independent of the HIP library: it shares no code with it and never
imports it. The arithmetic lives in attention.c (plain definition of attention in double
precision); this module only marshals numpy arrays through ctypes.

Parity pins (tests/test_oracle_*.py): a library routine (torch's CPU scaled-dot-product
attention in float64 with band masks built from tril), 50-digit mpmath brute force on tiny
inputs, closed forms (Q = 0 gives the mean of the visible V rows and LSE = ln(count)),
invariants (rows sum to one, shift and permutation invariance, split-and-merge of keys),
one-hot edge probes of every mask boundary, and reductions between masks (a band or prefix
covering every key is the unmasked case, an empty prefix is causal, an all-ones block layout
is unmasked). The gradients are pinned to torch autograd in float64, central finite
differences of the forward pass and the invariants of the softmax Jacobian, for the
block-sparse layout as for the masks.
"""
import ctypes
import os

import numpy as np

from . import build as _build


class Oracle:
    """ctypes handle on a built oracle library (the default one, or another build of the
    same source, as the mutation tests use)."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_attention_rows.argtypes = [
            f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_long, ctypes.c_long, i64p,
            ctypes.c_long, f64p, f64p]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_decode_paged.argtypes = [
            f32p, f32p, f32p, i32p, i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_double, f64p, f64p]
        lib.oracle_decode_paged.restype = ctypes.c_int
        lib.oracle_prefill_paged.argtypes = [
            f32p, f32p, f32p, i32p, i32p, i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_double,
            ctypes.c_int, ctypes.c_long, ctypes.c_long, f64p, f64p]
        lib.oracle_prefill_paged.restype = ctypes.c_int
        lib.oracle_attention_block_sparse_rows.argtypes = [
            f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_uint8), ctypes.c_long, i64p,
            ctypes.c_long, f64p, f64p]
        lib.oracle_attention_block_sparse_rows.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [
            f32p, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_long, ctypes.c_long, f64p,
            f64p, f64p]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_attention_backward_block_sparse.argtypes = [
            f32p, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_uint8), ctypes.c_long, f64p,
            f64p, f64p]
        lib.oracle_attention_backward_block_sparse.restype = ctypes.c_int
        lib.oracle_merge_lse.argtypes = [f32p, f32p, f32p, f32p, ctypes.c_long, ctypes.c_int,
                                         f64p, f64p]
        lib.oracle_merge_lse.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self):
        return int(self.lib.oracle_num_threads())

    def attention(self, q, k, v, scale, mask_mode=0, window=0, n_global=0, rows=None):
        """Exact attention in fp64.

        q: [B,H,Nq,d], k/v: [B,H,Nkv,d] (any float dtype; taken as exact float32 values).
        scale: the float32 scale the device receives (upcast exactly).
        rows: optional 1-D array of flat query-row indices ((b*H+h)*Nq + i).
        Returns (o, lse): o [B,H,Nq,d] (or [len(rows), d]) float64, lse [B,H,Nq] (or [len]).
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        assert k.shape == (B, H, Nkv, d) and v.shape == (B, H, Nkv, d)
        scale = float(np.float32(scale))
        if rows is None:
            n = B * H * Nq
            rp = None
        else:
            rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n = rows.size
            rp = _p(rows, ctypes.c_int64)
        o = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(
            _p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float), B, H, Nq,
            Nkv, d, scale, int(mask_mode), int(window), int(n_global), rp, n,
            _p(o, ctypes.c_double), _p(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_attention_rows rejected its arguments")
        if rows is None:
            return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)
        return o, lse

    def attention_backward(self, q, k, v, dout, scale, mask_mode=0, window=0, n_global=0):
        """Gradients (dq, dk, dv) of exact attention for upstream gradient dout, fp64.

        q, dout: [B,H,Nq,d]; k, v: [B,H,Nkv,d]. Returns float64 arrays of the same shapes.
        """
        q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        assert k.shape == (B, H, Nkv, d) and v.shape == k.shape and g.shape == q.shape
        dq = np.empty(q.shape, np.float64)
        dk = np.empty(k.shape, np.float64)
        dv = np.empty(k.shape, np.float64)
        rc = self.lib.oracle_attention_backward(
            _p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
            _p(g, ctypes.c_float), B, H, Nq, Nkv, d, float(np.float32(scale)), int(mask_mode),
            int(window), int(n_global), _p(dq, ctypes.c_double), _p(dk, ctypes.c_double),
            _p(dv, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_attention_backward rejected its arguments")
        return dq, dk, dv

    def attention_backward_block_sparse(self, q, k, v, dout, scale, layout, block):
        """Gradients (dq, dk, dv) of block-sparse attention (layout as in
        attention_block_sparse) for upstream gradient dout, fp64."""
        q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        assert k.shape == (B, H, Nkv, d) and v.shape == k.shape and g.shape == q.shape
        lay = np.ascontiguousarray(np.asarray(layout).astype(np.uint8))
        assert lay.shape == (H, -(-Nq // block), -(-Nkv // block)), lay.shape
        dq = np.empty(q.shape, np.float64)
        dk = np.empty(k.shape, np.float64)
        dv = np.empty(k.shape, np.float64)
        rc = self.lib.oracle_attention_backward_block_sparse(
            _p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
            _p(g, ctypes.c_float), B, H, Nq, Nkv, d, float(np.float32(scale)),
            _p(lay, ctypes.c_uint8), int(block), _p(dq, ctypes.c_double),
            _p(dk, ctypes.c_double), _p(dv, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_attention_backward_block_sparse rejected its arguments")
        return dq, dk, dv

    def attention_block_sparse(self, q, k, v, scale, layout, block, rows=None):
        """Exact block-sparse attention in fp64.

        layout: [H, ceil(Nq/block), ceil(Nkv/block)], nonzero = visible tile (shared by every
        batch entry). Other arguments and the result as in attention().
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        assert k.shape == (B, H, Nkv, d) and v.shape == (B, H, Nkv, d)
        lay = np.ascontiguousarray(np.asarray(layout).astype(np.uint8))
        assert lay.shape == (H, -(-Nq // block), -(-Nkv // block)), lay.shape
        scale = float(np.float32(scale))
        if rows is None:
            n = B * H * Nq
            rp = None
        else:
            rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n = rows.size
            rp = _p(rows, ctypes.c_int64)
        o = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self.lib.oracle_attention_block_sparse_rows(
            _p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float), B, H, Nq,
            Nkv, d, scale, _p(lay, ctypes.c_uint8), int(block), rp, n, _p(o, ctypes.c_double),
            _p(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_attention_block_sparse_rows rejected its arguments")
        if rows is None:
            return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)
        return o, lse

    def prefill_paged(self, q, k_pages, v_pages, page_table, seq_lens, q_lens, scale,
                      mask_mode=1, window=0, n_global=0):
        """Chunked prefill against a paged cache, fp64: q [S,Qmax,H,d], sequence s's chunk is
        its newest q_lens[s] tokens of seq_lens[s]. Returns (o [S,Qmax,H,d], lse [S,Qmax,H])
        float64, NaN in rows at or past q_lens[s]."""
        q, kp, vp = _f32(q), _f32(k_pages), _f32(v_pages)
        pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        ql = np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
        S, Qmax, H, d = q.shape
        num_pages, page_size = kp.shape[0], kp.shape[1]
        assert kp.shape == (num_pages, page_size, H, d) and vp.shape == kp.shape
        assert pt.shape[0] == S and sl.shape == (S,) and ql.shape == (S,)
        o = np.full((S, Qmax, H, d), np.nan, dtype=np.float64)
        lse = np.full((S, Qmax, H), np.nan, dtype=np.float64)
        rc = self.lib.oracle_prefill_paged(
            _p(q, ctypes.c_float), _p(kp, ctypes.c_float), _p(vp, ctypes.c_float),
            _p(pt, ctypes.c_int32), _p(sl, ctypes.c_int32), _p(ql, ctypes.c_int32), S, Qmax, H,
            d, page_size, pt.shape[1], num_pages, float(np.float32(scale)), int(mask_mode),
            int(window), int(n_global), _p(o, ctypes.c_double), _p(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_prefill_paged rejected its arguments")
        return o, lse

    def merge_lse(self, o_a, lse_a, o_b, lse_b):
        """Merge two attention results over disjoint key sets (same rows), fp64.

        o_*: [..., d]; lse_*: [...] (natural log). Returns (o, lse) float64 of those shapes.
        """
        oa, ob, la, lb = _f32(o_a), _f32(o_b), _f32(lse_a), _f32(lse_b)
        assert oa.shape == ob.shape and la.shape == lb.shape == oa.shape[:-1]
        d = oa.shape[-1]
        rows = int(np.prod(la.shape))
        o = np.empty(oa.shape, np.float64)
        lse = np.empty(la.shape, np.float64)
        self.lib.oracle_merge_lse(_p(oa, ctypes.c_float), _p(la, ctypes.c_float),
                                  _p(ob, ctypes.c_float), _p(lb, ctypes.c_float), rows, d,
                                  _p(o, ctypes.c_double), _p(lse, ctypes.c_double))
        return o, lse

    def multimodal(self, q_img, k_img, v_img, q_txt, k_txt, v_txt, scale):
        """Attention of one image-text sequence with the article's multimodal pattern, fp64:
        image tokens attend to all image tokens only; text tokens attend to all image tokens
        and causally to text tokens (ascend-transformer-boost article, 场景四). On the
        sequence [image; text] that is the prefix-LM mask with the image as the prefix, one
        call of the plain definition. Inputs [B,H,N_img|N_txt,d]. Returns (o_img, lse_img,
        o_txt, lse_txt) float64."""
        qi, ki, vi = _f32(q_img), _f32(k_img), _f32(v_img)
        qt, kt, vt = _f32(q_txt), _f32(k_txt), _f32(v_txt)
        n_img = qi.shape[2]
        q = np.concatenate([qi, qt], axis=2)
        k = np.concatenate([ki, kt], axis=2)
        v = np.concatenate([vi, vt], axis=2)
        o, lse = self.attention(q, k, v, scale, 4, 0, n_img)
        return o[:, :, :n_img], lse[:, :, :n_img], o[:, :, n_img:], lse[:, :, n_img:]

    def decode_paged(self, q, k_pages, v_pages, page_table, seq_lens, scale):
        """Single-token decode against a paged cache, fp64.

        q: [S,H,d]; k_pages/v_pages: [num_pages, page_size, H, d]; page_table:
        [S, max_pages] int32; seq_lens: [S] int32. Returns (o [S,H,d], lse [S,H]) float64.
        """
        q, kp, vp = _f32(q), _f32(k_pages), _f32(v_pages)
        pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        S, H, d = q.shape
        num_pages, page_size = kp.shape[0], kp.shape[1]
        assert kp.shape == (num_pages, page_size, H, d) and vp.shape == kp.shape
        assert pt.shape[0] == S and sl.shape == (S,)
        o = np.empty((S, H, d), dtype=np.float64)
        lse = np.empty((S, H), dtype=np.float64)
        rc = self.lib.oracle_decode_paged(
            _p(q, ctypes.c_float), _p(kp, ctypes.c_float), _p(vp, ctypes.c_float),
            _p(pt, ctypes.c_int32), _p(sl, ctypes.c_int32), S, H, d, page_size, pt.shape[1],
            num_pages, float(np.float32(scale)), _p(o, ctypes.c_double),
            _p(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_decode_paged rejected its arguments")
        return o, lse


def _f32(a):
    """Exact float32 view of the values the device receives (fp16/bf16/fp32 all fit)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float32).numpy()
    except ImportError:
        pass
    a = np.asarray(a)
    if a.dtype != np.float32:
        a = a.astype(np.float32)
    return np.ascontiguousarray(a)


def _p(a, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


_default = None


def default():
    """The oracle built from attention.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def num_threads():
    return default().num_threads()


def attention(*args, **kw):
    return default().attention(*args, **kw)


def attention_block_sparse(*args, **kw):
    return default().attention_block_sparse(*args, **kw)


def attention_backward_block_sparse(*args, **kw):
    return default().attention_backward_block_sparse(*args, **kw)


def attention_backward(*args, **kw):
    return default().attention_backward(*args, **kw)


def decode_paged(*args, **kw):
    return default().decode_paged(*args, **kw)


def prefill_paged(*args, **kw):
    return default().prefill_paged(*args, **kw)


def merge_lse(*args, **kw):
    return default().merge_lse(*args, **kw)


def multimodal(*args, **kw):
    return default().multimodal(*args, **kw)
