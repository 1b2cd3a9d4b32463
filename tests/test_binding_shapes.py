"""Host-side shape checks of the Python binding (CPU only: every mismatched tensor must be
rejected with ValueError before any pointer reaches the library, so no kernel can read or
write out of bounds on a GPU)."""
import pytest
import torch

import tiled_exact_attention_forward_amd as fa


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


I32 = torch.int32


@pytest.mark.parametrize("kw,match", [
    (dict(out=t(1, 2, 64, 128)), "out must have shape"),
    (dict(lse=t(1, 2, 64, dtype=torch.float32)), "lse must have shape"),
])
def test_forward_shapes(kw, match):
    q, k, v = t(1, 2, 65, 128), t(1, 2, 70, 128), t(1, 2, 70, 128)
    with pytest.raises(ValueError, match=match):
        fa.fa_forward(q, k, v, **kw)
    with pytest.raises(ValueError, match=match):
        fa.fa_forward_block_sparse(q, k, v, t(2, 1, 1, dtype=torch.uint8), **kw)


def test_forward_kv_shape():
    with pytest.raises(ValueError, match="k and v"):
        fa.fa_forward(t(1, 2, 65, 128), t(1, 2, 70, 128), t(1, 2, 71, 128))


@pytest.mark.parametrize("which,shape", [("dq", (1, 2, 64, 128)), ("dk", (1, 2, 65, 128)),
                                         ("dv", (1, 1, 70, 128))])
def test_backward_shapes(which, shape):
    q, k, v = t(1, 2, 65, 128), t(1, 2, 70, 128), t(1, 2, 70, 128)
    kw = {which: t(*shape)}
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        fa.fa_backward(q, k, v, t(1, 2, 65, 128), t(1, 2, 65, dtype=torch.float32),
                       t(1, 2, 65, 128), **kw)


def decode_args(**over):
    a = dict(q=t(3, 8, 128, dtype=torch.float16), k_pages=t(5, 256, 8, 128, dtype=torch.float16),
             v_pages=t(5, 256, 8, 128, dtype=torch.float16), page_table=t(3, 2, dtype=I32),
             seq_lens=t(3, dtype=I32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(k_pages=t(5, 256, 4, 128, dtype=torch.float16)), "k_pages must have shape"),
    (dict(v_pages=t(4, 256, 8, 128, dtype=torch.float16)), "v_pages must have shape"),
    (dict(page_table=t(2, 2, dtype=I32)), "page_table must be"),
    (dict(page_table=t(6, dtype=I32)), "page_table must be"),
    (dict(seq_lens=t(4, dtype=I32)), "seq_lens must have shape"),
    (dict(out=t(3, 8, 64, dtype=torch.float16)), "out must have shape"),
    (dict(lse=t(3, 4, dtype=torch.float32)), "lse must have shape"),
])
def test_decode_shapes(over, match):
    with pytest.raises(ValueError, match=match):
        fa.fa_decode_paged(**decode_args(**over))


def prefill_args(**over):
    a = dict(q=t(3, 40, 8, 128), k_pages=t(5, 256, 8, 128), v_pages=t(5, 256, 8, 128),
             page_table=t(3, 2, dtype=I32), seq_lens=t(3, dtype=I32), q_lens=t(3, dtype=I32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(k_pages=t(5, 256, 4, 128)), "k_pages and v_pages"),
    (dict(page_table=t(4, 2, dtype=I32)), "page_table must be"),
    (dict(seq_lens=t(2, dtype=I32)), "seq_lens must have shape"),
    (dict(q_lens=t(3, 1, dtype=I32)), "q_lens must have shape"),
    (dict(out=t(3, 40, 8, 64)), "out must have shape"),
    (dict(lse=t(3, 40, dtype=torch.float32)), "lse must have shape"),
])
def test_prefill_shapes(over, match):
    with pytest.raises(ValueError, match=match):
        fa.fa_prefill_paged(**prefill_args(**over))


def test_merge_shapes():
    oa, la = t(10, 128), t(10, dtype=torch.float32)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fa_merge_lse(oa, la, oa, la, out=t(9, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_merge_lse(oa, la, oa, la, lse=t(11, dtype=torch.float32))
