"""Helpers for the GPU parity tests: device transfer and tolerances.

Tolerances (stated once, used by every GPU parity test):
  * fp16 / bf16 outputs: max |O_gpu - O_ref| <= 1e-2 over every compared element and
    max |LSE_gpu - LSE_ref| <= 1e-3 (the stated bar). Because that bar is loose for
    outputs of size ~0.05, the relative L2 error ||O_gpu - O_ref|| / ||O_ref|| is also gated:
    <= 8e-3 (bf16) and <= 2e-3 (fp16). Rounding P and O to the 16-bit type each adds a
    relative error of at most 2^-9 (bf16) / 2^-12 (fp16), i.e. about 2e-3 / 2.5e-4 rms.
  * fp32: normwise relative, max |O_gpu - O_ref| <= 1e-5 * max |O_ref|, and
    |LSE_gpu - LSE_ref| <= 1e-5 * max(1, |LSE_ref|).
The reference is the fp64 oracle on exactly the values the GPU received; it is not rounded
to the output type (the tolerance absorbs that rounding).
"""
import numpy as np
import torch

import oracle

O_ABS = 1e-2
LSE_ABS = 1e-3
REL_L2 = {"bf16": 8e-3, "f16": 2e-3}
F32_REL = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def to_dev(*ts):
    dev = require_gpu()
    return [t.to(dev).contiguous() for t in ts]


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    og, lg = f64(o_gpu), f64(lse_gpu)
    o_ref = np.asarray(o_ref, np.float64).reshape(og.shape)
    lse_ref = np.asarray(lse_ref, np.float64).reshape(lg.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), "LSE finiteness differs"
    diff = np.abs(og - o_ref)
    worst = np.unravel_index(int(np.argmax(diff)), diff.shape) if diff.size else ()
    return dict(
        o_max_abs=float(diff.max()) if diff.size else 0.0,
        o_worst_at=tuple(int(x) for x in worst),
        o_ref_max=float(np.abs(o_ref).max()) if o_ref.size else 0.0,
        o_rel_l2=float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300)),
        lse_max_abs=float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0,
        lse_rel=float((np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1, np.abs(lse_ref[fin]))).max())
        if fin.any() else 0.0,
        nan=bool(np.isnan(og).any() or np.isnan(lg[fin]).any()),
    )


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    e = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    assert not e["nan"], f"{label}: NaN in output {e}"
    if dtype == "f32":
        assert e["o_max_abs"] <= F32_REL * e["o_ref_max"], f"{label}: {e}"
        assert e["lse_rel"] <= F32_REL, f"{label}: {e}"
    else:
        assert e["o_max_abs"] <= O_ABS, f"{label}: {e}"
        assert e["lse_max_abs"] <= LSE_ABS, f"{label}: {e}"
        assert e["o_rel_l2"] <= REL_L2[dtype], f"{label}: {e}"
    return e


# Unit roundoff of the 16-bit types, for the gradient tolerances below. The float32 backward
# rounds nothing to 16 bits; its error comes from float32 sums over the rows or keys a
# gradient element collects (random-sign rounding errors grow like sqrt(N) 2^-24: 2^-18 at
# N = 4096, 2^-15 at the longest sequence the entry points take, 2^18) and from
# P = 2^(c s - L), whose exponent carries the forward's LSE error (~2^-20 in practice):
# u = 2^-16 puts the rel-L2 gate 4u at 2^-14, twice the longest sum's expected error
# (measured: 2^-20 at N <= 1500, 2^-17 at 2^18 rows).
U_GRAD = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -16}


def check_grads(got, ref, dtype, label, inputs, scale, vis):
    """Gradients (dq, dk, dv) against the oracle's, with the backward's tolerance (stated in
    test_backward_gpu's docstring): max-abs within 8u of each tensor's largest reference
    value plus the float32 accumulation floor, rel-L2 within 4u, structural zeros exact.
    inputs = (q, k, v, do) as given to both sides; vis = bool [Nq, Nkv] visibility, or the
    pair (rows without a visible key, keys no row sees) already taken from it."""
    u = U_GRAD[dtype]
    q, k, v, do = (float(t.float().abs().max()) for t in inputs)
    d = inputs[0].shape[-1]
    fl = abs(scale) * 2 * d * 2.0 ** -20 * do * v * max(q, k)
    if isinstance(vis, tuple):
        zero_rows, zero_keys = vis
    else:
        zero_rows = ~vis.any(dim=1).numpy()  # [Nq]
        zero_keys = ~vis.any(dim=0).numpy()  # [Nkv]
    out = {}
    for name, g, r, floor in zip(("dq", "dk", "dv"), got, ref, (fl, fl, 0.0)):
        g = f64(g)
        r = np.asarray(r, np.float64).reshape(g.shape)
        assert not np.isnan(g).any(), f"{label}: NaN in {name}"
        diff = np.abs(g - r)
        rmax = float(np.abs(r).max()) if r.size else 0.0
        mabs = float(diff.max()) if diff.size else 0.0
        rl2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        out[name] = (mabs, rmax, rl2)
        assert mabs <= 8 * u * rmax + floor, f"{label}: {name} max-abs {mabs} ref max {rmax}"
        if rmax > 64 * floor:
            assert rl2 <= 4 * u, f"{label}: {name} rel-L2 {rl2}"
        structural = zero_rows if name == "dq" else zero_keys
        assert np.all(g[:, :, structural] == 0.0), f"{label}: {name} nonzero at a structural 0"
    return out
