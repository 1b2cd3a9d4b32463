"""Python binding of libteaf.so, the MI355X (gfx950) tiled exact attention library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in include/fa.h. The functions carry the C names:

    fa_forward(q, k, v, ...)          tiled exact attention forward (O and LSE)
    fa_forward_block_sparse(...)      forward with a block-sparse layout of visible tiles
    fa_backward(q, k, v, o, lse, dout, ...)  gradients dQ, dK, dV
    fa_backward_block_sparse(...)     gradients of the block-sparse forward
    fa_backward_workspace_bytes(...)
    fa_decode_paged(q, k_pages, ...)  single-token decode against a paged K/V cache
    fa_decode_paged_noalloc(...)      the same without a workspace (library's static scratch)
    fa_prefill_paged(q, k_pages, ...) multi-token chunk per sequence against a paged cache
    fa_merge_lse(o_a, lse_a, o_b, lse_b, ...)  merge results over disjoint key sets
    fa_multimodal_forward(...)        image/text attention as three calls plus a merge
    fa_multimodal_workspace_bytes(...)
    fa_decode_paged_workspace_bytes(...)
    fa_status_string(status)

Tensors are torch tensors on the GPU (torch supplies device memory and the current stream);
they are passed to the library as raw device pointers. There is no fallback: if the library
has not been built, importing the binding's functions raises.
"""
import ctypes
import math
import os

__all__ = ["fa_forward", "fa_forward_block_sparse", "fa_backward", "fa_backward_block_sparse",
           "fa_backward_workspace_bytes",
           "fa_decode_paged", "fa_decode_paged_noalloc", "fa_prefill_paged", "fa_merge_lse", "fa_multimodal_forward",
           "fa_multimodal_workspace_bytes", "fa_decode_paged_workspace_bytes",
           "fa_status_string", "fa_last_hip_error", "fa_version", "FaError", "library_path", "load_library",
           "FA_F32", "FA_F16", "FA_BF16", "FA_MASK_NONE", "FA_MASK_CAUSAL",
           "FA_MASK_WINDOW_GLOBAL", "FA_MASK_BAND", "FA_MASK_PREFIX_LM", "FA_MULTIMODAL_SPLIT_MERGE",
           "FA_MULTIMODAL_FUSED", "EXPORTED_SYMBOLS"]

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
FA_ERR_SCRATCH = -6
FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_WINDOW_GLOBAL, FA_MASK_BAND, FA_MASK_PREFIX_LM = 0, 1, 2, 3, 4
FA_MULTIMODAL_SPLIT_MERGE, FA_MULTIMODAL_FUSED = 0, 1
EXPORTED_SYMBOLS = ("fa_forward", "fa_forward_block_sparse", "fa_backward",
                    "fa_backward_block_sparse", "fa_backward_workspace_bytes", "fa_decode_paged", "fa_decode_paged_noalloc",
                    "fa_prefill_paged",
                    "fa_merge_lse", "fa_multimodal_forward", "fa_multimodal_workspace_bytes",
                    "fa_decode_paged_workspace_bytes", "fa_status_string", "fa_last_hip_error",
                    "fa_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path():
    return os.path.join(_HERE, "libteaf.so")


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {fa_status_string(status)} (status {status})"
        if status == FA_ERR_HIP:
            msg += f": {fa_last_hip_error()}"
        super().__init__(msg)


def load_library():
    """Load libteaf.so (raises if it was not built: there is no other code path)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- load torch's HIP runtime first so the library shares it
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -m tiled_exact_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_block_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, i, vp]
    lib.fa_forward_block_sparse.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i,
                                vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                             f, vp, i, i, vp, sz, vp]
    lib.fa_backward_block_sparse.restype = i
    lib.fa_decode_paged_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_paged_workspace_bytes.restype = sz
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz,
                                    vp]
    lib.fa_decode_paged.restype = i
    lib.fa_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                                            vp]
    lib.fa_decode_paged_noalloc.restype = i
    lib.fa_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i,
                                     i, i, i, vp]
    lib.fa_prefill_paged.restype = i
    lib.fa_merge_lse.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_longlong, i, i, vp]
    lib.fa_merge_lse.restype = i
    lib.fa_multimodal_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_multimodal_workspace_bytes.restype = sz
    lib.fa_multimodal_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                          f, i, i, vp, sz, vp]
    lib.fa_multimodal_forward.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.restype = i
    lib.fa_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def fa_last_hip_error():
    return load_library().fa_last_hip_error().decode()


def fa_version():
    return int(load_library().fa_version())


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    m = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_shape(name, t, shape):
    """Host-side shape check (before any pointer reaches the library)."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def fa_forward(q, k, v, scale=None, mask_mode=FA_MASK_NONE, window=0, n_global=0, out=None,
               lse=None, stream=None):
    """O, LSE = attention(q, k, v) with q [B,H,Nq,d], k/v [B,H,Nkv,d] (f32/f16/bf16).

    scale defaults to the float32 value of 1/sqrt(d). Returns (out, lse) with out like q and
    lse float32 [B,H,Nq]. Runs asynchronously on `stream` (torch's current stream if None).
    """
    torch = _torch()
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if tuple(k.shape) != (B, H, Nkv, d) or tuple(v.shape) != (B, H, Nkv, d):
        raise ValueError("k and v must be [B,H,Nkv,d] matching q")
    _check_shape("out", out, q.shape)
    _check_shape("lse", lse, (B, H, Nq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    rc = load_library().fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq,
                                   Nkv, d, float(scale), int(mask_mode), int(window),
                                   int(n_global), _dtype_code(q), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_forward")
    return out, lse


def fa_forward_block_sparse(q, k, v, layout, block=128, scale=None, out=None, lse=None,
                            stream=None):
    """Block-sparse attention: layout is a uint8 GPU tensor [H, ceil(Nq/block),
    ceil(Nkv/block)] (nonzero = visible tile), shared by every batch entry. Other arguments
    and the result as fa_forward."""
    torch = _torch()
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if tuple(k.shape) != (B, H, Nkv, d) or tuple(v.shape) != (B, H, Nkv, d):
        raise ValueError("k and v must be [B,H,Nkv,d] matching q")
    want = (H, -(-Nq // block), -(-Nkv // block))
    if tuple(layout.shape) != want or not layout.is_contiguous():
        raise ValueError(f"layout must be a contiguous {want} tensor")
    _check_shape("out", out, q.shape)
    _check_shape("lse", lse, (B, H, Nq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    _check_dev("layout", layout, torch.uint8)
    rc = load_library().fa_forward_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nkv, d, float(scale),
        _ptr(layout), int(block), _dtype_code(q), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_forward_block_sparse")
    return out, lse


def fa_backward_workspace_bytes(B, H, Nq):
    return int(load_library().fa_backward_workspace_bytes(int(B), int(H), int(Nq)))


def _backward_args(q, k, v, o, lse, dout, dq, dk, dv, workspace):
    """Shape and device checks shared by the backward calls; allocates what is missing."""
    torch = _torch()
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if tuple(k.shape) != (B, H, Nkv, d) or tuple(v.shape) != (B, H, Nkv, d):
        raise ValueError("k and v must be [B,H,Nkv,d] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be [B,H,Nq]")
    _check_shape("dq", dq, q.shape)
    _check_shape("dk", dk, k.shape)
    _check_shape("dv", dv, v.shape)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fa_backward_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    _check_dev("workspace", workspace)
    return dq, dk, dv, workspace


def fa_backward(q, k, v, o, lse, dout, scale=None, mask_mode=FA_MASK_NONE, window=0,
                n_global=0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of fa_forward: q [B,H,Nq,d], k/v [B,H,Nkv,d] (f32/f16/bf16), o and lse the
    forward's outputs for the same arguments, dout like o. Returns (dq, dk, dv)."""
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    dq, dk, dv, workspace = _backward_args(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = load_library().fa_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), B, H, Nq, Nkv, d, float(scale), int(mask_mode), int(window), int(n_global),
        _dtype_code(q), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_backward")
    return dq, dk, dv


def fa_backward_block_sparse(q, k, v, o, lse, dout, layout, block=128, scale=None, dq=None,
                             dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of fa_forward_block_sparse (same layout and block); other arguments and
    the result as fa_backward."""
    torch = _torch()
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    want = (H, -(-Nq // block), -(-Nkv // block))
    if tuple(layout.shape) != want or not layout.is_contiguous():
        raise ValueError(f"layout must be a contiguous {want} tensor")
    dq, dk, dv, workspace = _backward_args(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    _check_dev("layout", layout, torch.uint8)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = load_library().fa_backward_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), B, H, Nq, Nkv, d, float(scale), _ptr(layout), int(block), _dtype_code(q),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_backward_block_sparse")
    return dq, dk, dv


def fa_decode_paged_workspace_bytes(num_seqs, H, d, max_pages_per_seq, page_size=256):
    return int(load_library().fa_decode_paged_workspace_bytes(
        int(num_seqs), int(H), int(d), int(max_pages_per_seq), int(page_size)))


def _check_decode_shapes(q, k_pages, v_pages, page_table, seq_lens, out, lse):
    S, H, d = q.shape
    if k_pages.dim() != 4:
        raise ValueError("k_pages must be [num_pages, page_size, H, d]")
    P, page_size = k_pages.shape[0], k_pages.shape[1]
    _check_shape("k_pages", k_pages, (P, page_size, H, d))
    _check_shape("v_pages", v_pages, (P, page_size, H, d))
    if page_table.dim() != 2 or page_table.shape[0] != S:
        raise ValueError(f"page_table must be [{S}, max_pages_per_seq], got "
                         f"{tuple(page_table.shape)}")
    _check_shape("seq_lens", seq_lens, (S,))
    _check_shape("out", out, (S, H, d))
    _check_shape("lse", lse, (S, H))


def fa_decode_paged_noalloc(q, k_pages, v_pages, page_table, seq_lens, scale=None, out=None,
                            lse=None, stream=None):
    """fa_decode_paged with the split partials in the library's static scratch (no
    workspace). `out` and `lse` should be given by callers that must not allocate; calls
    on one GPU must not overlap. Returns (out, lse)."""
    torch = _torch()
    _check_decode_shapes(q, k_pages, v_pages, page_table, seq_lens, out, lse)
    S, H, d = q.shape
    P, page_size = k_pages.shape[0], k_pages.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("out", out)):
        _check_dev(name, t, q.dtype)
    _check_dev("page_table", page_table, torch.int32)
    _check_dev("seq_lens", seq_lens, torch.int32)
    _check_dev("lse", lse, torch.float32)
    rc = load_library().fa_decode_paged_noalloc(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(seq_lens), _ptr(out),
        _ptr(lse), page_size, S, H, d, page_table.shape[1], P, float(scale), _dtype_code(q),
        _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_decode_paged_noalloc")
    return out, lse


def fa_decode_paged(q, k_pages, v_pages, page_table, seq_lens, scale=None, out=None, lse=None,
                    workspace=None, stream=None):
    """Single-token decode: q [S,H,d]; pages [P,page_size,H,d]; page_table [S,max_pages]
    int32; seq_lens [S] int32 (all on the GPU). Returns (out [S,H,d], lse [S,H] float32)."""
    torch = _torch()
    _check_decode_shapes(q, k_pages, v_pages, page_table, seq_lens, out, lse)
    S, H, d = q.shape
    P, page_size = k_pages.shape[0], k_pages.shape[1]
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    need = fa_decode_paged_workspace_bytes(S, H, d, max_pages, page_size)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("out", out)):
        _check_dev(name, t, q.dtype)
    _check_dev("page_table", page_table, torch.int32)
    _check_dev("seq_lens", seq_lens, torch.int32)
    _check_dev("lse", lse, torch.float32)
    _check_dev("workspace", workspace)
    rc = load_library().fa_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(seq_lens), _ptr(out),
        _ptr(lse), page_size, S, H, d, max_pages, P, float(scale), _dtype_code(q),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_decode_paged")
    return out, lse


def fa_prefill_paged(q, k_pages, v_pages, page_table, seq_lens, q_lens, scale=None,
                     mask_mode=FA_MASK_CAUSAL, window=0, n_global=0, out=None, lse=None,
                     stream=None):
    """Chunked prefill: q [S,Qmax,H,d] holds each sequence's newest q_lens[s] tokens of its
    seq_lens[s] cached ones; pages [P,256,H,d]; page_table [S,max_pages] int32; seq_lens and
    q_lens [S] int32 (all on the GPU). Returns (out [S,Qmax,H,d], lse [S,Qmax,H] float32);
    rows at or past q_lens[s] are left as they were in `out` and `lse`."""
    torch = _torch()
    S, Qmax, H, d = q.shape
    P, page_size = k_pages.shape[0], k_pages.shape[1]
    if tuple(k_pages.shape) != (P, page_size, H, d) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages and v_pages must be [num_pages, page_size, H, d]")
    if page_table.dim() != 2 or page_table.shape[0] != S:
        raise ValueError(f"page_table must be [{S}, max_pages_per_seq], got "
                         f"{tuple(page_table.shape)}")
    _check_shape("seq_lens", seq_lens, (S,))
    _check_shape("q_lens", q_lens, (S,))
    _check_shape("out", out, (S, Qmax, H, d))
    _check_shape("lse", lse, (S, Qmax, H))
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    if lse is None:
        lse = torch.full((S, Qmax, H), float("-inf"), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("out", out)):
        _check_dev(name, t, q.dtype)
    for name, t in (("page_table", page_table), ("seq_lens", seq_lens), ("q_lens", q_lens)):
        _check_dev(name, t, torch.int32)
    _check_dev("lse", lse, torch.float32)
    rc = load_library().fa_prefill_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(seq_lens), _ptr(q_lens),
        _ptr(out), _ptr(lse), page_size, S, Qmax, H, d, max_pages, P, float(scale),
        int(mask_mode), int(window), int(n_global), _dtype_code(q), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_prefill_paged")
    return out, lse


def fa_merge_lse(o_a, lse_a, o_b, lse_b, out=None, lse=None, stream=None):
    """Merge attention results over disjoint key sets: o_* [..., d], lse_* [...] float32
    (GPU). Returns (out, lse); out/lse may be o_a/lse_a for an in-place merge."""
    torch = _torch()
    d = o_a.shape[-1]
    if tuple(o_b.shape) != tuple(o_a.shape) or tuple(lse_a.shape) != tuple(o_a.shape[:-1]) \
            or tuple(lse_b.shape) != tuple(lse_a.shape):
        raise ValueError("o_a, o_b [..., d] and lse_a, lse_b [...] must match")
    _check_shape("out", out, o_a.shape)
    _check_shape("lse", lse, lse_a.shape)
    out = torch.empty_like(o_a) if out is None else out
    lse = torch.empty_like(lse_a) if lse is None else lse
    for name, t in (("o_a", o_a), ("o_b", o_b), ("out", out)):
        _check_dev(name, t, o_a.dtype)
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b), ("lse", lse)):
        _check_dev(name, t, torch.float32)
    rc = load_library().fa_merge_lse(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out),
                                     _ptr(lse), lse_a.numel(), d, _dtype_code(o_a),
                                     _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_merge_lse")
    return out, lse


def fa_multimodal_workspace_bytes(B, H, n_txt, d, dtype_code):
    return int(load_library().fa_multimodal_workspace_bytes(int(B), int(H), int(n_txt), int(d),
                                                            int(dtype_code)))


def fa_multimodal_forward(q_img, k_img, v_img, q_txt, k_txt, v_txt, scale=None,
                          text_mode=FA_MULTIMODAL_SPLIT_MERGE, workspace=None, stream=None):
    """Image/text attention (image sees image; text sees image and earlier text). text_mode
    FA_MULTIMODAL_SPLIT_MERGE: three attention calls and a log-sum-exp merge;
    FA_MULTIMODAL_FUSED: the image call and one causal call over [image; text] keys read from
    the two tensors (n_img % 32 == 0, fp16/bf16). Inputs [B,H,n,d] on the GPU. Returns
    (o_img, lse_img, o_txt, lse_txt)."""
    torch = _torch()
    B, H, n_img, d = q_img.shape
    n_txt = q_txt.shape[2]
    for name, t, n in (("k_img", k_img, n_img), ("v_img", v_img, n_img),
                       ("q_txt", q_txt, n_txt), ("k_txt", k_txt, n_txt),
                       ("v_txt", v_txt, n_txt)):
        if tuple(t.shape) != (B, H, n, d):
            raise ValueError(f"{name} must be [B,H,{n},d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_img, o_txt = torch.empty_like(q_img), torch.empty_like(q_txt)
    lse_img = torch.empty((B, H, n_img), dtype=torch.float32, device=q_img.device)
    lse_txt = torch.empty((B, H, n_txt), dtype=torch.float32, device=q_img.device)
    code = _dtype_code(q_img)
    need = fa_multimodal_workspace_bytes(B, H, n_txt, d, code)
    if workspace is None and text_mode == FA_MULTIMODAL_SPLIT_MERGE:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q_img.device)
    for name, t in (("q_img", q_img), ("k_img", k_img), ("v_img", v_img), ("q_txt", q_txt),
                    ("k_txt", k_txt), ("v_txt", v_txt)):
        _check_dev(name, t, q_img.dtype)
    _check_dev("workspace", workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().fa_multimodal_forward(
        _ptr(q_img), _ptr(k_img), _ptr(v_img), _ptr(q_txt), _ptr(k_txt), _ptr(v_txt),
        _ptr(o_img), _ptr(lse_img), _ptr(o_txt), _ptr(lse_txt), B, H, n_img, n_txt, d,
        float(scale), code, int(text_mode), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_multimodal_forward")
    return o_img, lse_img, o_txt, lse_txt
