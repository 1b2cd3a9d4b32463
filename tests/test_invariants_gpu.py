"""Properties of the HIP path that hold exactly or by construction, plus checker sensitivity.

* V = 1 gives O = 1 (rows of P sum to one), for every mask.
* Q = 0 gives LSE = ln(count of visible keys), with the count from its closed form.
* Causal (and window) row 0 equals V[0] exactly.
* One-hot probes: a dominant score on one key returns that key's V row when the mask shows
  it, and the mean of the visible rows when it hides it, at every mask edge and across the
  64-key tile boundary.
* Out-of-range memory is never read: NaN placed right after K/V (prefill) and in unused
  page slots and spare pages (decode) does not reach the output.
* Paged decode is independent of the physical page placement (bit-identical), agrees with
  the forward pass on the same keys, and the forward pass with one query agrees with the
  last row of the causal square case.
* Two runs give bit-identical results (no atomics in any reduction).
* Sensitivity: the GPU output FAILS the parity check against oracle builds with a planted
  mistake, so the tolerances can see each of those mistakes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import pins
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check, errors, f64, require_gpu, to_dev
from mutants import build_mutant

pytestmark = pytest.mark.gpu


def fwd(q, k, v, scale, mask=0, W=0, G=0):
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fa_forward(qd, kd, vd, scale, mask, W, G)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mask", [(0, 0, 0), (1, 0, 0), (2, 50, 7), (3, 20, 0), (4, 0, 70)])
def test_rows_sum_to_one(dtype, mask):
    q, k, _ = workloads.gen_prefill(2, 3, 200, 200, 128, dtype, 11)
    v = torch.ones_like(q)
    o, _ = fwd(q, k, v, 0.0884, *mask)
    tol = 1e-6 if dtype == "f32" else 2 ** -7
    assert (f64(o) - 1).__abs__().max() <= tol


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("shape,mask", [((300, 300), (0, 0, 0)), ((300, 300), (1, 0, 0)),
                                        ((150, 300), (1, 0, 0)), ((300, 300), (2, 70, 9)),
                                        ((257, 257), (2, 1, 0)), ((200, 300), (2, 64, 130)),
                                        ((300, 300), (3, 45, 0)), ((150, 300), (3, 7, 0)),
                                        ((300, 150), (3, 100, 0)), ((300, 300), (4, 0, 100)),
                                        ((150, 300), (4, 0, 200)), ((300, 150), (4, 0, 40))])
def test_q_zero_gives_log_count(dtype, shape, mask):
    Nq, Nkv = shape
    _, k, v = workloads.gen_prefill(1, 2, Nq, Nkv, 64, dtype, 12)
    q = torch.zeros((1, 2, Nq, 64), dtype=k.dtype)
    o, lse = fwd(q, k, v, 0.125, *mask)
    counts = np.array([pins.visible_count(i + Nkv - Nq, Nkv, mask[0], mask[1], mask[2])
                       for i in range(Nq)])
    lg = f64(lse)
    seen = counts > 0
    lc = np.log(counts[seen])
    assert np.abs(lg[:, :, seen] - lc[None, None, :]).max() <= 2e-6 * lc.max() + 1e-6
    assert np.all(np.isneginf(lg[:, :, ~seen]))  # rows without a visible key
    ro, rl = oracle.attention(q, k, v, 0.125, *mask)
    check(o, lse, ro, rl, dtype, "q=0")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mask", [(1, 0, 0), (2, 16, 4)])
def test_first_row_is_first_value(dtype, mask):
    q, k, v = workloads.gen_prefill(2, 4, 130, 130, 128, dtype, 13)
    o, lse = fwd(q, k, v, 0.0884, *mask)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_onehot_edge_probes(dtype):
    N, d, W, G = 128, 128, 16, 8
    # row: key carrying the dominant score; edges at the diagonal, the window start and
    # end, the global boundary and the 64-key tile boundary
    probes = {63: 63, 64: 64, 65: 66, 79: 64, 80: 64, 100: 7, 101: 8, 127: 112, 126: 110,
              5: 5, 6: 7, 70: 55, 71: 55}
    q, k, v = pins.onehot_case(N, d, W, G, list(probes.items()), c=8.0, alpha=40.0)
    t = workloads.DTYPES[dtype]
    q, k, v = torch.from_numpy(q).to(t), torch.from_numpy(k).to(t), torch.from_numpy(v).to(t)
    o, lse = fwd(q, k, v, 0.125, 2, W, G)
    ro, rl = oracle.attention(q, k, v, 0.125, 2, W, G)
    check(o, lse, ro, rl, dtype, "onehot")
    og, vf = f64(o)[0, 0], f64(v)[0, 0]
    for i, j in probes.items():
        keys = pins.visible_keys(i, N, 2, W, G)
        want = vf[j] if j in keys else vf[keys].mean(axis=0)
        other = vf[keys].mean(axis=0) if j in keys else vf[j]
        assert np.abs(og[i] - want).max() < 1e-2, (i, j)
        assert np.abs(og[i] - other).max() > 5e-2, (i, j)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("mask", [(3, 16, 0), (4, 0, 16)])
def test_onehot_edge_probes_band_prefix(dtype, mask):
    N, d = 128, 128
    mode, W, G = mask
    if mode == 3:  # band +-16: both edges, across 32-key tile boundaries
        probes = {40: 56, 41: 58, 60: 44, 61: 44, 0: 16, 1: 18, 127: 111, 126: 109, 31: 47,
                  33: 16}
    else:          # prefix of 16 keys: the prefix edge from early rows, the diagonal later
        probes = {0: 15, 1: 16, 2: 2, 3: 4, 63: 63, 64: 65, 100: 15, 101: 17, 127: 127}
    q, k, v = pins.onehot_case(N, d, W, G, list(probes.items()), c=8.0, alpha=40.0)
    t = workloads.DTYPES[dtype]
    q, k, v = torch.from_numpy(q).to(t), torch.from_numpy(k).to(t), torch.from_numpy(v).to(t)
    o, lse = fwd(q, k, v, 0.125, mode, W, G)
    ro, rl = oracle.attention(q, k, v, 0.125, mode, W, G)
    check(o, lse, ro, rl, dtype, f"onehot mode {mode}")
    og, vf = f64(o)[0, 0], f64(v)[0, 0]
    for i, j in probes.items():
        keys = pins.visible_keys(i, N, mode, W, G)
        want = vf[j] if j in keys else vf[keys].mean(axis=0)
        other = vf[keys].mean(axis=0) if j in keys else vf[j]
        assert np.abs(og[i] - want).max() < 1e-2, (i, j)
        assert np.abs(og[i] - other).max() > 5e-2, (i, j)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mask", [(0, 0, 0), (1, 0, 0), (2, 30, 3), (3, 40, 0), (4, 0, 60)])
def test_never_reads_past_the_keys(dtype, mask):
    dev = require_gpu()
    B, H, Nq, Nkv, d = 1, 2, 150, 100, 128
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, 14)
    n = k.numel()
    pad = 64 * 128 * 4
    ks = torch.full((n + pad,), float("nan"), dtype=k.dtype, device=dev)
    vs = torch.full((n + pad,), float("nan"), dtype=k.dtype, device=dev)
    ks[:n] = k.reshape(-1).to(dev)
    vs[:n] = v.reshape(-1).to(dev)
    kd, vd = ks[:n].view(k.shape), vs[:n].view(v.shape)
    qd = q.to(dev)
    o, lse = fa.fa_forward(qd, kd, vd, 0.0884, *mask)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, 0.0884, *mask)
    check(o, lse, ro, rl, dtype, "nan canary")


def _decode(inp, scale):
    q, kp, vp, pt, sl = to_dev(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                               inp["seq_lens"])
    o, lse = fa.fa_decode_paged(q, kp, vp, pt, sl, scale)
    torch.cuda.synchronize()
    return o, lse


def _repage(inp, seed):
    """Same logical cache, different physical placement (and more spare NaN pages)."""
    rng = np.random.default_rng(seed)
    kp, vp, pt, sl = inp["k_pages"], inp["v_pages"], inp["page_table"].numpy(), inp["seq_lens"]
    used = pt[pt >= 0]
    total = kp.shape[0] + 3
    newid = rng.permutation(total)[:used.size]
    kn = torch.full((total,) + tuple(kp.shape[1:]), float("nan"), dtype=kp.dtype)
    vn = torch.full_like(kn, float("nan"))
    pt2 = np.full_like(pt, -1)
    n = 0
    for s in range(pt.shape[0]):
        for p in range(pt.shape[1]):
            if pt[s, p] >= 0:
                kn[newid[n]] = kp[pt[s, p]]
                vn[newid[n]] = vp[pt[s, p]]
                pt2[s, p] = newid[n]
                n += 1
    return dict(inp, k_pages=kn, v_pages=vn, page_table=torch.from_numpy(pt2))


def test_decode_page_placement_is_bit_invariant():
    _, inp = workloads.gen_workload("decode_f16", S=4, lens=[300, 5000, 256, 8192])
    o1, l1 = _decode(inp, 0.0884)
    o2, l2 = _decode(_repage(inp, 3), 0.0884)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_matches_forward_and_causal_last_row(dtype):
    lens = [700, 64, 1, 2049]
    _, inp = workloads.gen_workload("decode_f16", dtype=dtype, S=len(lens), H=8, lens=lens)
    o, lse = _decode(inp, 0.0884)
    pt, kp, vp = inp["page_table"], inp["k_pages"], inp["v_pages"]
    for s, L in enumerate(lens):
        ids = [int(pt[s, j // 256]) for j in range(L)]
        slots = [j % 256 for j in range(L)]
        kc = kp[ids, slots].permute(1, 0, 2).unsqueeze(0).contiguous()  # [1,H,L,d]
        vc = vp[ids, slots].permute(1, 0, 2).unsqueeze(0).contiguous()
        q1 = inp["q"][s].unsqueeze(0).unsqueeze(2).contiguous()  # [1,H,1,d]
        of, lf = fwd(q1, kc, vc, 0.0884, 0)
        assert np.abs(f64(of)[0, :, 0] - f64(o)[s]).max() < 1e-2
        assert np.abs(f64(lf)[0, :, 0] - f64(lse)[s]).max() < 1e-3
        # causal square case: the last row sees every key
        qq = torch.cat([kc[:, :, :L - 1], q1], dim=2).contiguous()
        oc, lc = fwd(qq, kc, vc, 0.0884, 1)
        assert np.abs(f64(oc)[0, :, L - 1] - f64(o)[s]).max() < 1e-2
        assert np.abs(f64(lc)[0, :, L - 1] - f64(lse)[s]).max() < 1e-3


@pytest.mark.parametrize("mask", [(0, 0, 0), (1, 0, 0), (2, 100, 10), (3, 300, 0), (4, 0, 500)])
def test_bitwise_deterministic(mask):
    q, k, v = workloads.gen_prefill(2, 4, 700, 700, 128, "bf16", 15)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.fa_forward(qd, kd, vd, 0.0884, *mask)
    o2, l2 = fa.fa_forward(qd, kd, vd, 0.0884, *mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _, inp = workloads.gen_workload("decode_f16", S=3, lens=[4000, 100, 8000])
    a = _decode(inp, 0.0884)
    b = _decode(inp, 0.0884)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


SENSITIVITY = {
    "causal_strict": dict(mask=(1, 0, 0), shape=(200, 200)),
    "window_inclusive": dict(mask=(2, 40, 5), shape=(300, 300)),
    "global_inclusive": dict(mask=(2, 40, 5), shape=(300, 300)),
    "top_left_causal": dict(mask=(1, 0, 0), shape=(100, 300)),
    "no_normalise": dict(mask=(0, 0, 0), shape=(100, 100)),
    "scale_dropped": dict(mask=(0, 0, 0), shape=(100, 100)),
    "lse_drops_max": dict(mask=(0, 0, 0), shape=(100, 100)),
    "value_as_key": dict(mask=(0, 0, 0), shape=(100, 100)),
    "page_slot": dict(decode=True),
    "decode_head": dict(decode=True),
}


@pytest.mark.parametrize("name", sorted(SENSITIVITY))
def test_checker_rejects_planted_mistakes(name, tmp_path):
    cfg = SENSITIVITY[name]
    bad = build_mutant(name, str(tmp_path))
    if cfg.get("decode"):
        _, inp = workloads.gen_workload("decode_f16", S=3, H=8, lens=[600, 4000, 70])
        o, lse = _decode(inp, 0.0884)
        ro, rl = bad.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], 0.0884)
        go, gl = oracle.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"],
                                     inp["page_table"], inp["seq_lens"], 0.0884)
    else:
        Nq, Nkv = cfg["shape"]
        q, k, v = workloads.gen_prefill(1, 4, Nq, Nkv, 128, "bf16", 16)
        o, lse = fwd(q, k, v, 0.0884, *cfg["mask"])
        ro, rl = bad.attention(q, k, v, 0.0884, *cfg["mask"])
        go, gl = oracle.attention(q, k, v, 0.0884, *cfg["mask"])
    check(o, lse, go, gl, "bf16" if not cfg.get("decode") else "f16", "good oracle")
    with pytest.raises(AssertionError):
        check(o, lse, ro, rl, "bf16" if not cfg.get("decode") else "f16", f"mutant {name}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("mask", [(0, 0, 0), (1, 0, 0), (2, 70, 0), (3, 20, 0)])
@pytest.mark.parametrize("slope", [0.5, 3.0, 40.0])
def test_rising_scores_rescale(dtype, mask, slope):
    """Scores that grow from key tile to key tile, so that a later tile's probabilities
    against the reference taken from an earlier tile overflow every bound (fp16 P tops out
    at 65504) unless the running maximum is raised: q . k_j = slope * j / 32 (natural units
    after the scale), plus noise. Compared with the oracle over several query tiles, with
    rows whose first visible key lies past their first key tile (band and window masks)."""
    N, d = 300, 128
    g = torch.Generator("cpu").manual_seed(int(slope * 10) + 7 * mask[0])
    q = torch.zeros((1, 2, N, d))
    k = torch.randn((1, 2, N, d), generator=g) * 0.05
    v = torch.randn((1, 2, N, d), generator=g) * 0.25  # |O| < 1, as the 1e-2 bound assumes
    q[..., 0] = 1.0
    k[..., 0] += slope * torch.arange(N, dtype=torch.float32) / 32 * 8.0  # scale 1/8
    t = workloads.DTYPES[dtype]
    q, k, v = q.to(t), k.to(t), v.to(t)
    o, lse = fwd(q, k, v, 0.125, *mask)
    ro, rl = oracle.attention(q, k, v, 0.125, *mask)
    check(o, lse, ro, rl, dtype, f"rising {dtype} {mask} slope {slope}")
