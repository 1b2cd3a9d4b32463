"""Pins of the fp64 oracle to facts other than itself.

Each pin takes an oracle handle (oracle.default() or a deliberately broken build of the same
source) and raises AssertionError when the oracle disagrees with:
  * a library routine: torch's CPU scaled_dot_product_attention and logsumexp in float64,
    with the masks built from torch.tril band offsets rather than from an index predicate;
  * 50-digit mpmath brute force over explicitly enumerated key sets on tiny inputs;
  * closed forms: Q = 0 makes every visible score equal, so O is the mean of the visible V
    rows (computed from prefix sums) and LSE = ln(count), with count from its own formula;
  * invariants: rows sum to one (V = 1 gives O = 1), a common score shift moves LSE only,
    jointly permuting keys and values changes nothing (no mask), attention over a key split
    merged by log-sum-exp equals attention over all keys (the multimodal split in the
    "ascend-transformer-boost" article, 场景四, is stated to be numerically identical);
  * one-hot probes that put a dominant score on one key and check which V row comes out, at
    every mask edge: the causal diagonal, the key after it, the first and last key of the
    window, the last global key and the key after it.
The backward oracle is pinned to torch autograd in float64, to central finite differences of
the oracle's own forward pass, and to exact invariants of the softmax Jacobian.
Masks: 0 none, 1 causal (diagonal kept, aligned bottom-right), 2 causal window of W keys
ending at the query plus the first G keys, 3 band of W positions on both sides of the query,
4 prefix LM (the first G keys visible to every query, the rest causal); block sparse takes a
per-head layout of block x block tiles.
"""
import math

import numpy as np
import torch

RNG_SEED = 1234


def _rand(shape, seed, dtype=np.float32):
    return np.random.default_rng(seed).standard_normal(shape).astype(dtype)


def band_mask(Nq, Nkv, mode, W=0, G=0):
    """Boolean [Nq, Nkv] visibility built from tril band offsets (True = visible)."""
    delta = Nkv - Nq
    ones = torch.ones(Nq, Nkv, dtype=torch.bool)
    if mode == 0:
        return ones
    causal = torch.tril(ones, diagonal=delta)
    if mode == 1:
        return causal
    if mode == 3:
        return torch.tril(ones, diagonal=delta + W) & ~torch.tril(ones, diagonal=delta - W - 1)
    if mode == 4:
        prefix = torch.zeros(Nq, Nkv, dtype=torch.bool)
        prefix[:, :G] = True
        return causal | prefix
    window = causal & ~torch.tril(ones, diagonal=delta - W)
    glob = causal.clone()
    glob[:, G:] = False
    return window | glob


def block_mask(layout, block, Nq, Nkv):
    """Boolean [H, Nq, Nkv] visibility of a block layout, expanded with a Kronecker product."""
    lay = torch.from_numpy(np.asarray(layout, dtype=np.int64))
    tile = torch.ones(block, block, dtype=torch.int64)
    full = torch.stack([torch.kron(lay[h], tile) for h in range(lay.shape[0])])
    return full[:, :Nq, :Nkv] != 0


def library_attention_mask(q, k, v, scale, m):
    """torch SDPA + logsumexp in float64 with an explicit boolean mask (broadcast)."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~m, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def library_attention(q, k, v, scale, mode, W=0, G=0):
    """torch SDPA + logsumexp in float64 on the CPU (rows with no visible key excluded)."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    m = band_mask(qt.shape[-2], kt.shape[-2], mode, W, G)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), m.numpy()


def visible_keys(ip, Nkv, mode, W, G):
    """Explicit visible key set for a query at absolute position ip (range arithmetic)."""
    if mode == 0:
        return list(range(Nkv))
    hi = min(ip, Nkv - 1)
    if hi < 0 and mode in (1, 2):
        return []
    if mode == 1:
        return list(range(0, hi + 1))
    if mode == 3:
        return list(range(max(0, ip - W), min(Nkv - 1, ip + W) + 1))
    if mode == 4:
        return sorted(set(range(0, hi + 1)) | set(range(0, min(G, Nkv))))
    win = set(range(max(0, ip - W + 1), hi + 1))
    glob = set(range(0, min(G, hi + 1)))
    return sorted(win | glob)


def visible_count(ip, Nkv, mode, W, G):
    """Closed-form count of visible keys (no enumeration)."""
    if mode == 0:
        return Nkv
    if mode == 3:
        return max(0, min(Nkv - 1, ip + W) - max(0, ip - W) + 1)
    if mode == 4:
        return min(Nkv, max(G, ip + 1, 0))
    if ip < 0:
        return 0
    top = min(ip, Nkv - 1) + 1
    if mode == 1:
        return top
    start = max(0, ip - W + 1)
    in_win = max(0, top - start)
    return in_win + max(0, min(G, start, top))


def mp_attention_row(q, krows, vrows, scale, keys):
    import mpmath as mp
    with mp.workdps(50):
        sc = mp.mpf(float(scale))
        s = {j: sc * mp.fsum(mp.mpf(float(a)) * mp.mpf(float(b)) for a, b in zip(q, krows[j]))
             for j in keys}
        m = max(s.values())
        e = {j: mp.exp(s[j] - m) for j in keys}
        l = mp.fsum(e.values())
        o = [mp.fsum(e[j] * mp.mpf(float(vrows[j][c])) for j in keys) / l
             for c in range(len(q))]
        return [float(x) for x in o], float(m + mp.log(l))


# --------------------------------------------------------------------------- pins

def pin_library(orc):
    cases = [(1, 1, 9, 9, 8, 0, 0, 0), (2, 3, 17, 17, 16, 1, 0, 0), (1, 2, 33, 33, 8, 2, 5, 3),
             (1, 2, 40, 40, 4, 2, 1, 0), (1, 1, 12, 30, 8, 1, 0, 0), (1, 1, 12, 30, 8, 2, 7, 2),
             (1, 2, 25, 25, 64, 2, 30, 40), (2, 1, 20, 20, 8, 0, 0, 0)]
    for n, (B, H, Nq, Nkv, d, mode, W, G) in enumerate(cases):
        q = _rand((B, H, Nq, d), RNG_SEED + 3 * n)
        k = _rand((B, H, Nkv, d), RNG_SEED + 3 * n + 1)
        v = _rand((B, H, Nkv, d), RNG_SEED + 3 * n + 2)
        scale = float(np.float32(1 / math.sqrt(d)))
        o, lse = orc.attention(q, k, v, scale, mode, W, G)
        ro, rl, _ = library_attention(q, k, v, scale, mode, W, G)
        assert np.allclose(o, ro, rtol=1e-12, atol=1e-13), f"library O mismatch case {n}"
        assert np.allclose(lse, rl, rtol=1e-12, atol=1e-13), f"library LSE mismatch case {n}"


def pin_mpmath(orc):
    cases = [(1, 1, 1, 1, 0, 0, 0), (3, 3, 4, 1, 0, 0), (7, 7, 4, 2, 2, 1), (7, 7, 4, 2, 5, 3),
             (4, 7, 2, 1, 0, 0), (5, 5, 1, 0, 0, 0), (6, 6, 8, 2, 1, 0), (16, 16, 4, 2, 5, 3)]
    for n, case in enumerate(cases):
        Nq, Nkv, d, mode, W, G = case[0], case[1], case[2], case[3], case[4], case[5]
        q = _rand((1, 1, Nq, d), 77 + n) * 2
        k = _rand((1, 1, Nkv, d), 177 + n) * 2
        v = _rand((1, 1, Nkv, d), 277 + n)
        scale = 0.7
        o, lse = orc.attention(q, k, v, scale, mode, W, G)
        for i in range(Nq):
            keys = visible_keys(i + Nkv - Nq, Nkv, mode, W, G)
            ro, rl = mp_attention_row(q[0, 0, i], k[0, 0], v[0, 0], np.float32(scale), keys)
            assert np.allclose(o[0, 0, i], ro, rtol=1e-12, atol=1e-14), (n, i)
            assert abs(lse[0, 0, i] - rl) <= 1e-12 * max(1.0, abs(rl)), (n, i)


def pin_q_zero(orc):
    for n, (Nq, Nkv, mode, W, G) in enumerate([(50, 50, 0, 0, 0), (50, 50, 1, 0, 0),
                                               (20, 50, 1, 0, 0), (60, 60, 2, 8, 5),
                                               (60, 60, 2, 1, 0), (40, 70, 2, 16, 20),
                                               (30, 30, 2, 40, 2)]):
        d = 8
        q = np.zeros((1, 2, Nq, d), np.float32)
        k = _rand((1, 2, Nkv, d), 500 + n)
        v = _rand((1, 2, Nkv, d), 600 + n).astype(np.float64).astype(np.float32)
        o, lse = orc.attention(q, k, v, 0.3, mode, W, G)
        pre = np.concatenate([np.zeros((1, 2, 1, d)), np.cumsum(v.astype(np.float64), axis=2)],
                             axis=2)
        for i in range(Nq):
            ip = i + Nkv - Nq
            cnt = visible_count(ip, Nkv, mode, W, G)
            assert abs(lse[0, :, i] - math.log(cnt)).max() < 1e-12, (n, i)
            if mode == 0:
                tot = pre[0, :, Nkv]
            elif mode == 1:
                tot = pre[0, :, ip + 1]
            else:
                start = max(0, ip - W + 1)
                g_end = min(G, start)
                tot = pre[0, :, ip + 1] - pre[0, :, start] + pre[0, :, g_end]
            assert np.allclose(o[0, :, i], tot / cnt, rtol=1e-12, atol=1e-13), (n, i)


def pin_causal_row0(orc):
    for n, mode in enumerate([1, 2]):
        q = _rand((2, 2, 30, 16), 700 + n)
        k = _rand((2, 2, 30, 16), 710 + n)
        v = _rand((2, 2, 30, 16), 720 + n)
        scale = 0.25
        o, lse = orc.attention(q, k, v, scale, mode, 4, 2)
        assert np.array_equal(o[:, :, 0], v[:, :, 0].astype(np.float64)), "row 0 != V[0]"
        dot = np.einsum("bhc,bhc->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
        assert np.allclose(lse[:, :, 0], scale * dot, rtol=1e-13, atol=1e-14)


def onehot_case(N, d, W, G, probes, c=8.0, alpha=8.0):
    """K rows c*e_j (orthogonal, needs N <= d); Q rows alpha*e_{j*} for each probe (i, j*)."""
    assert N <= d
    k = np.zeros((1, 1, N, d), np.float32)
    for j in range(N):
        k[0, 0, j, j] = c
    q = np.zeros((1, 1, N, d), np.float32)
    for i, js in probes:
        q[0, 0, i, js] = alpha
    v = _rand((1, 1, N, d), 900)
    return q, k, v


def pin_onehot_edges(orc):
    N, d, W, G = 48, 64, 8, 4
    probes = {
        # row: (probe key, expected visible?)
        20: (20, True),          # causal diagonal
        21: (22, False),         # the key after the diagonal
        30: (30 - W + 1, True),  # first key inside the window
        31: (31 - W, False),     # the key just outside the window (not global)
        40: (G - 1, True),       # last global key, far outside the window
        41: (G, False),          # first non-global key, outside the window
        10: (10 - W + 1, True),
        2: (2, True),
    }
    q, k, v = onehot_case(N, d, W, G, [(i, js) for i, (js, _) in probes.items()])
    scale = 1.0 / 8.0  # alpha*c*scale = 8 per dominant score -> mass on one key >= 1-1e-...
    q *= 5  # dominant score 40 (e^-40 ~ 4e-18 leakage)
    o, lse = orc.attention(q, k, v, scale, 2, W, G)
    for i, (js, vis) in probes.items():
        keys = visible_keys(i, N, 2, W, G)
        if vis:
            assert js in keys
            assert np.allclose(o[0, 0, i], v[0, 0, js], rtol=0, atol=1e-12), (i, js)
            assert abs(lse[0, 0, i] - (40.0 + math.log1p((len(keys) - 1) * math.exp(-40.0)))) < 1e-12
        else:
            assert js not in keys
            mean = v[0, 0, keys].astype(np.float64).mean(axis=0)
            assert np.allclose(o[0, 0, i], mean, rtol=1e-12, atol=1e-13), (i, js)
            assert abs(lse[0, 0, i] - math.log(len(keys))) < 1e-12
    # causal mode: the diagonal is visible, the key after it is not
    q2, k2, v2 = onehot_case(N, d, W, G, [(5, 5), (6, 7)])
    q2 *= 5
    o2, _ = orc.attention(q2, k2, v2, scale, 1)
    assert np.allclose(o2[0, 0, 5], v2[0, 0, 5], atol=1e-12)
    assert np.allclose(o2[0, 0, 6], v2[0, 0, :7].astype(np.float64).mean(axis=0), atol=1e-12)
    # no mask: a dominant key past the diagonal is still selected
    o3, _ = orc.attention(q2, k2, v2, scale, 0)
    assert np.allclose(o3[0, 0, 6], v2[0, 0, 7], atol=1e-12)


def pin_rows_sum_to_one(orc):
    for mode in (0, 1, 2):
        q = _rand((1, 3, 40, 16), 1000 + mode) * 3
        k = _rand((1, 3, 40, 16), 1010 + mode) * 3
        v = np.ones((1, 3, 40, 16), np.float32)
        o, _ = orc.attention(q, k, v, 0.5, mode, 5, 3)
        assert np.allclose(o, 1.0, rtol=0, atol=1e-14)


def pin_shift(orc):
    d, N = 16, 25
    q = _rand((1, 2, N, d), 1100)
    k = _rand((1, 2, N, d), 1101)
    v = _rand((1, 2, N, d), 1102)
    scale = 0.25
    for mode in (0, 1, 2):
        o0, l0 = orc.attention(q, k, v, scale, mode, 6, 2)
        for c in (-800.0, 800.0):
            qe = np.float32(c / scale)
            q2 = np.concatenate([q, np.full((1, 2, N, 1), qe, np.float32)], axis=-1)
            k2 = np.concatenate([k, np.ones((1, 2, N, 1), np.float32)], axis=-1)
            v2 = np.concatenate([v, np.zeros((1, 2, N, 1), np.float32)], axis=-1)
            o1, l1 = orc.attention(q2, k2, v2, scale, mode, 6, 2)
            shift = scale * float(qe)
            assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
            assert np.allclose(o1[..., :d], o0, rtol=1e-10, atol=1e-10)
            assert np.allclose(l1 - shift, l0, rtol=0, atol=1e-9)


def pin_permutation(orc):
    q = _rand((2, 2, 19, 8), 1200)
    k = _rand((2, 2, 31, 8), 1201)
    v = _rand((2, 2, 31, 8), 1202)
    perm = np.random.default_rng(5).permutation(31)
    o0, l0 = orc.attention(q, k, v, 0.4, 0)
    o1, l1 = orc.attention(q, k[:, :, perm], v[:, :, perm], 0.4, 0)
    assert np.allclose(o0, o1, rtol=1e-13, atol=1e-14)
    assert np.allclose(l0, l1, rtol=1e-13, atol=1e-14)


def pin_split_merge(orc):
    q = _rand((1, 2, 13, 8), 1300) * 2
    k = _rand((1, 2, 40, 8), 1301) * 2
    v = _rand((1, 2, 40, 8), 1302)
    o, l = orc.attention(q, k, v, 0.6, 0)
    oa, la = orc.attention(q, k[:, :, :17], v[:, :, :17], 0.6, 0)
    ob, lb = orc.attention(q, k[:, :, 17:], v[:, :, 17:], 0.6, 0)
    lm = np.logaddexp(la, lb)
    om = np.exp(la - lm)[..., None] * oa + np.exp(lb - lm)[..., None] * ob
    assert np.allclose(lm, l, rtol=1e-13, atol=1e-13)
    assert np.allclose(om, o, rtol=1e-12, atol=1e-13)


def pin_mask_reductions(orc):
    q = _rand((1, 2, 24, 8), 1400)
    k = _rand((1, 2, 24, 8), 1401)
    v = _rand((1, 2, 24, 8), 1402)
    oc, lc = orc.attention(q, k, v, 0.35, 1)
    for W, G in ((24, 0), (1000, 3), (1, 24), (5, 1000)):
        ow, lw = orc.attention(q, k, v, 0.35, 2, W, G)
        assert np.array_equal(ow, oc) and np.array_equal(lw, lc), (W, G)
    o1, l1 = orc.attention(q, k[:, :, :1], v[:, :, :1], 0.35, 0)
    assert np.array_equal(o1, np.broadcast_to(v[:, :, :1].astype(np.float64), o1.shape))
    # window of one key and no global keys: every row sees only itself
    ow, _ = orc.attention(q, k, v, 0.35, 2, 1, 0)
    assert np.array_equal(ow, v.astype(np.float64))


def pin_empty_rows(orc):
    # more queries than keys with bottom-right causal: the first Nq-Nkv rows see nothing
    q = _rand((1, 1, 10, 8), 1500)
    k = _rand((1, 1, 4, 8), 1501)
    v = _rand((1, 1, 4, 8), 1502)
    o, l = orc.attention(q, k, v, 0.35, 1)
    assert np.all(o[0, 0, :6] == 0) and np.all(np.isneginf(l[0, 0, :6]))
    assert np.array_equal(o[0, 0, 6], v[0, 0, 0].astype(np.float64))
    assert np.all(np.isfinite(l[0, 0, 6:]))


def make_paged(k, v, page_size, seed, spare=2):
    """Scatter contiguous per-sequence K/V [S][L_s,H,d] into a permuted page pool."""
    rng = np.random.default_rng(seed)
    S = len(k)
    H, d = k[0].shape[1], k[0].shape[2]
    npg = [(x.shape[0] + page_size - 1) // page_size for x in k]
    total = sum(npg) + spare
    perm = rng.permutation(total)
    kp = np.full((total, page_size, H, d), np.nan, np.float32)
    vp = np.full((total, page_size, H, d), np.nan, np.float32)
    pt = np.full((S, max(npg)), -1, np.int32)
    n = 0
    for s in range(S):
        for p in range(npg[s]):
            pid = perm[n]
            n += 1
            pt[s, p] = pid
            seg_k = k[s][p * page_size:(p + 1) * page_size]
            kp[pid, :seg_k.shape[0]] = seg_k
            vp[pid, :seg_k.shape[0]] = v[s][p * page_size:(p + 1) * page_size]
    return kp, vp, pt


def pin_decode(orc):
    H, d, ps = 3, 8, 16
    lens = [1, 16, 17, 40, 64]
    q = _rand((len(lens), H, d), 1600)
    ks = [_rand((L, H, d), 1610 + i) for i, L in enumerate(lens)]
    vs = [_rand((L, H, d), 1620 + i) for i, L in enumerate(lens)]
    kp, vp, pt = make_paged(ks, vs, ps, 7)
    o, l = orc.decode_paged(q, kp, vp, pt, np.array(lens, np.int32), 0.3)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    for s, L in enumerate(lens):
        # contiguous [1,H,L,d] against the same query: same result as the paged lookup
        kc = np.ascontiguousarray(ks[s].transpose(1, 0, 2))[None]
        vc = np.ascontiguousarray(vs[s].transpose(1, 0, 2))[None]
        ro, rl, _ = library_attention(q[s][None, :, None, :], kc, vc, float(np.float32(0.3)), 0)
        assert np.allclose(o[s], ro[0, :, 0], rtol=1e-12, atol=1e-13), s
        assert np.allclose(l[s], rl[0, :, 0], rtol=1e-12, atol=1e-13), s
    # a different physical placement gives bit-identical results
    kp2, vp2, pt2 = make_paged(ks, vs, ps, 8, spare=5)
    o2, l2 = orc.decode_paged(q, kp2, vp2, pt2, np.array(lens, np.int32), 0.3)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def _random_layout(H, nqb, nkb, seed, density=0.35):
    lay = (np.random.default_rng(seed).random((H, nqb, nkb)) < density).astype(np.uint8)
    lay[:, :, 0] |= (np.arange(nqb) % 3 == 0).astype(np.uint8)  # some rows with block 0
    return lay


def pin_library_more_masks(orc):
    """Band (3), prefix LM (4) and block sparse against torch SDPA with masks built by tril
    offsets and Kronecker products."""
    cases = [(1, 2, 33, 33, 8, 3, 4, 0), (1, 1, 12, 30, 8, 3, 6, 0), (2, 2, 25, 25, 16, 3, 0, 0),
             (1, 2, 33, 33, 8, 4, 0, 9), (1, 1, 12, 30, 8, 4, 0, 20), (1, 1, 30, 12, 8, 4, 0, 5),
             (2, 1, 20, 20, 8, 4, 0, 0), (1, 1, 40, 40, 4, 3, 100, 0)]
    for n, (B, H, Nq, Nkv, d, mode, W, G) in enumerate(cases):
        q = _rand((B, H, Nq, d), 3000 + 3 * n)
        k = _rand((B, H, Nkv, d), 3001 + 3 * n)
        v = _rand((B, H, Nkv, d), 3002 + 3 * n)
        scale = float(np.float32(1 / math.sqrt(d)))
        o, lse = orc.attention(q, k, v, scale, mode, W, G)
        ro, rl = library_attention_mask(q, k, v, scale, band_mask(Nq, Nkv, mode, W, G))
        assert np.allclose(o, ro, rtol=1e-12, atol=1e-13), f"library O mismatch case {n}"
        assert np.allclose(lse, rl, rtol=1e-12, atol=1e-13), f"library LSE mismatch case {n}"
    for n, (B, H, Nq, Nkv, d, blk) in enumerate([(1, 2, 40, 40, 8, 8), (2, 3, 33, 50, 8, 16),
                                                 (1, 1, 7, 64, 4, 4)]):
        q = _rand((B, H, Nq, d), 3100 + 3 * n)
        k = _rand((B, H, Nkv, d), 3101 + 3 * n)
        v = _rand((B, H, Nkv, d), 3102 + 3 * n)
        lay = _random_layout(H, -(-Nq // blk), -(-Nkv // blk), 3200 + n)
        m = block_mask(lay, blk, Nq, Nkv)[None]
        rows = m.any(dim=-1)[0]
        o, lse = orc.attention_block_sparse(q, k, v, 0.4, lay, blk)
        ro, rl = library_attention_mask(q, k, v, float(np.float32(0.4)), m)
        for h in range(H):
            vis = rows[h].numpy()
            assert np.allclose(o[:, h][:, vis], ro[:, h][:, vis], rtol=1e-12, atol=1e-13), n
            assert np.allclose(lse[:, h][:, vis], rl[:, h][:, vis], rtol=1e-12, atol=1e-13), n
            assert np.all(o[:, h][:, ~vis] == 0) and np.all(np.isneginf(lse[:, h][:, ~vis])), n


def pin_mpmath_more_masks(orc):
    for n, (Nq, Nkv, d, mode, W, G) in enumerate([(7, 7, 4, 3, 2, 0), (5, 9, 4, 3, 1, 0),
                                                 (9, 5, 4, 3, 3, 0), (7, 7, 4, 4, 0, 3),
                                                 (4, 9, 2, 4, 0, 2), (9, 4, 2, 4, 0, 2)]):
        q = _rand((1, 1, Nq, d), 3300 + n) * 2
        k = _rand((1, 1, Nkv, d), 3400 + n) * 2
        v = _rand((1, 1, Nkv, d), 3500 + n)
        o, lse = orc.attention(q, k, v, 0.7, mode, W, G)
        for i in range(Nq):
            keys = visible_keys(i + Nkv - Nq, Nkv, mode, W, G)
            if not keys:
                assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i]), (n, i)
                continue
            ro, rl = mp_attention_row(q[0, 0, i], k[0, 0], v[0, 0], np.float32(0.7), keys)
            assert np.allclose(o[0, 0, i], ro, rtol=1e-12, atol=1e-14), (n, i)
            assert abs(lse[0, 0, i] - rl) <= 1e-12 * max(1.0, abs(rl)), (n, i)
    # block sparse: key sets enumerated from the layout row
    blk, Nq, Nkv, d = 3, 8, 10, 4
    lay = np.array([[[1, 0, 1, 0], [0, 1, 0, 1], [1, 1, 0, 0]]], np.uint8)
    q = _rand((1, 1, Nq, d), 3600) * 2
    k = _rand((1, 1, Nkv, d), 3601) * 2
    v = _rand((1, 1, Nkv, d), 3602)
    o, lse = orc.attention_block_sparse(q, k, v, 0.7, lay, blk)
    for i in range(Nq):
        keys = [j for j in range(Nkv) if lay[0, i // blk, j // blk]]
        ro, rl = mp_attention_row(q[0, 0, i], k[0, 0], v[0, 0], np.float32(0.7), keys)
        assert np.allclose(o[0, 0, i], ro, rtol=1e-12, atol=1e-14), i
        assert abs(lse[0, 0, i] - rl) <= 1e-12 * max(1.0, abs(rl)), i


def pin_q_zero_more_masks(orc):
    for n, (Nq, Nkv, mode, W, G) in enumerate([(50, 50, 3, 7, 0), (30, 60, 3, 5, 0),
                                               (60, 30, 3, 2, 0), (50, 50, 4, 0, 13),
                                               (20, 50, 4, 0, 40), (50, 20, 4, 0, 6)]):
        d = 8
        q = np.zeros((1, 2, Nq, d), np.float32)
        k = _rand((1, 2, Nkv, d), 3700 + n)
        v = _rand((1, 2, Nkv, d), 3800 + n)
        o, lse = orc.attention(q, k, v, 0.3, mode, W, G)
        pre = np.concatenate([np.zeros((1, 2, 1, d)), np.cumsum(v.astype(np.float64), axis=2)],
                             axis=2)
        for i in range(Nq):
            ip = i + Nkv - Nq
            cnt = visible_count(ip, Nkv, mode, W, G)
            if cnt == 0:
                assert np.all(o[0, :, i] == 0) and np.all(np.isneginf(lse[0, :, i])), (n, i)
                continue
            assert abs(lse[0, :, i] - math.log(cnt)).max() < 1e-12, (n, i)
            if mode == 3:
                a, b = max(0, ip - W), min(Nkv - 1, ip + W) + 1
            else:
                a, b = 0, min(Nkv, max(G, ip + 1))
            tot = pre[0, :, b] - pre[0, :, a]
            assert np.allclose(o[0, :, i], tot / cnt, rtol=1e-12, atol=1e-13), (n, i)


def pin_onehot_more_edges(orc):
    N, d, scale = 48, 64, 1.0 / 8.0
    W = 5
    # band: i+W and i-W visible, i+W+1 and i-W-1 not
    probes = {20: (25, True), 21: (27, False), 30: (25, True), 31: (25, False), 0: (5, True),
              47: (42, True), 1: (7, False)}
    q, k, v = onehot_case(N, d, W, 0, [(i, js) for i, (js, _) in probes.items()])
    q *= 5
    o, lse = orc.attention(q, k, v, scale, 3, W, 0)
    for i, (js, vis) in probes.items():
        keys = visible_keys(i, N, 3, W, 0)
        assert (js in keys) == vis, (i, js)
        want = v[0, 0, js] if vis else v[0, 0, keys].astype(np.float64).mean(axis=0)
        assert np.allclose(o[0, 0, i], want, rtol=1e-12, atol=1e-12), ("band", i, js)
    # prefix LM with P = 10: row 0 sees key 9 but not key 10; row 20 sees 20, not 21
    P = 10
    probes = {0: (9, True), 1: (10, False), 20: (20, True), 21: (22, False), 3: (8, True)}
    q, k, v = onehot_case(N, d, 0, P, [(i, js) for i, (js, _) in probes.items()])
    q *= 5
    o, lse = orc.attention(q, k, v, scale, 4, 0, P)
    for i, (js, vis) in probes.items():
        keys = visible_keys(i, N, 4, 0, P)
        assert (js in keys) == vis, (i, js)
        want = v[0, 0, js] if vis else v[0, 0, keys].astype(np.float64).mean(axis=0)
        assert np.allclose(o[0, 0, i], want, rtol=1e-12, atol=1e-12), ("prefix", i, js)
    # block sparse, block 8: row 9 (query block 1) probes key 16 (block 2, set) and key 8
    # (block 1, not set); row 17 (block 2) probes key 7 (block 0, set) and 24 (block 3, not)
    lay = np.zeros((1, 6, 6), np.uint8)
    lay[0, 1, 2] = lay[0, 1, 0] = 1
    lay[0, 2, 0] = lay[0, 2, 2] = 1
    q, k, v = onehot_case(N, d, 0, 0, [(9, 16), (10, 8), (17, 7), (18, 24)])
    q *= 5
    o, _ = orc.attention_block_sparse(q, k, v, scale, lay, 8)
    both = np.r_[0:8, 16:24]
    assert np.allclose(o[0, 0, 9], v[0, 0, 16], atol=1e-12)
    assert np.allclose(o[0, 0, 10], v[0, 0, both].astype(np.float64).mean(axis=0), atol=1e-12)
    assert np.allclose(o[0, 0, 17], v[0, 0, 7], atol=1e-12)
    assert np.allclose(o[0, 0, 18], v[0, 0, both].astype(np.float64).mean(axis=0), atol=1e-12)
    assert np.all(o[0, 0, 0:8] == 0)  # query block 0 has no visible tile


def pin_more_mask_reductions(orc):
    q = _rand((1, 2, 24, 8), 3900)
    k = _rand((1, 2, 24, 8), 3901)
    v = _rand((1, 2, 24, 8), 3902)
    on, ln = orc.attention(q, k, v, 0.35, 0)
    oc, lc = orc.attention(q, k, v, 0.35, 1)
    for W in (23, 24, 1000):   # a band reaching every key is the unmasked case
        ob, lb = orc.attention(q, k, v, 0.35, 3, W, 0)
        assert np.array_equal(ob, on) and np.array_equal(lb, ln), W
    ob, _ = orc.attention(q, k, v, 0.35, 3, 0, 0)   # band of width 0: each row sees itself
    assert np.array_equal(ob, v.astype(np.float64))
    op, lp = orc.attention(q, k, v, 0.35, 4, 0, 0)  # empty prefix: causal
    assert np.array_equal(op, oc) and np.array_equal(lp, lc)
    for P in (24, 50):                               # prefix covering every key: unmasked
        op, lp = orc.attention(q, k, v, 0.35, 4, 0, P)
        assert np.array_equal(op, on) and np.array_equal(lp, ln), P
    for blk in (4, 7, 24, 32):                       # all-ones layout: unmasked
        lay = np.ones((2, -(-24 // blk), -(-24 // blk)), np.uint8)
        ob, lb = orc.attention_block_sparse(q, k, v, 0.35, lay, blk)
        assert np.array_equal(ob, on) and np.array_equal(lb, ln), blk


# --------------------------------------------------------------------------- backward

def library_backward(q, k, v, dout, scale, m):
    """Gradients from torch autograd through an explicit float64 softmax attention."""
    qt, kt, vt = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (q, k, v))
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~m, float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1))  # rows without a key: zeros
    torch.matmul(p, vt).backward(torch.tensor(np.asarray(dout, np.float64)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_backward_library(orc):
    cases = [(1, 2, 13, 17, 8, 0, 0, 0), (2, 1, 20, 20, 8, 1, 0, 0), (1, 2, 25, 12, 4, 1, 0, 0),
             (1, 1, 30, 30, 8, 2, 5, 3), (1, 2, 19, 26, 8, 3, 4, 0), (1, 1, 22, 22, 16, 4, 0, 6)]
    for n, (B, H, Nq, Nkv, d, mode, W, G) in enumerate(cases):
        q = _rand((B, H, Nq, d), 4000 + 4 * n)
        k = _rand((B, H, Nkv, d), 4001 + 4 * n)
        v = _rand((B, H, Nkv, d), 4002 + 4 * n)
        g = _rand((B, H, Nq, d), 4003 + 4 * n)
        scale = float(np.float32(1 / math.sqrt(d)))
        got = orc.attention_backward(q, k, v, g, scale, mode, W, G)
        want = library_backward(q, k, v, g, scale, band_mask(Nq, Nkv, mode, W, G))
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert np.allclose(a, b, rtol=1e-11, atol=1e-12), (n, name, np.abs(a - b).max())


def pin_backward_finite_difference(orc):
    """Central differences of L = sum(O * dO) computed by the oracle's own forward pass, with
    steps of 2^-10 that are exact in float32 around the inputs used."""
    h = 2.0 ** -10
    for n, (Nq, Nkv, d, mode, W, G) in enumerate([(5, 6, 3, 0, 0, 0), (6, 6, 3, 1, 0, 0),
                                                 (7, 7, 2, 3, 1, 0), (6, 6, 2, 4, 0, 2),
                                                 (7, 7, 2, 2, 2, 1)]):
        rng = np.random.default_rng(4100 + n)
        q, k, v, g = (np.round(rng.standard_normal(sh) * 64) / 64
                      for sh in ((1, 1, Nq, d), (1, 1, Nkv, d), (1, 1, Nkv, d), (1, 1, Nq, d)))
        q, k, v, g = (x.astype(np.float32) for x in (q, k, v, g))
        dq, dk, dv = orc.attention_backward(q, k, v, g, 0.5, mode, W, G)

        def loss(qq, kk, vv):
            o, _ = orc.attention(qq, kk, vv, 0.5, mode, W, G)
            return float((o * g.astype(np.float64)).sum())

        for which, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros(x.shape)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += np.float32(h)
                xm[idx] -= np.float32(h)
                if which == "q":
                    num[idx] = (loss(xp, k, v) - loss(xm, k, v)) / (2 * h)
                elif which == "k":
                    num[idx] = (loss(q, xp, v) - loss(q, xm, v)) / (2 * h)
                else:
                    num[idx] = (loss(q, k, xp) - loss(q, k, xm)) / (2 * h)
            assert np.allclose(grad, num, rtol=1e-5, atol=2e-6), (n, which,
                                                                  np.abs(grad - num).max())


def pin_backward_invariants(orc):
    """Each row's softmax Jacobian annihilates constants: sum_j dS_ij = 0, so dK summed over
    keys is zero; and P rows sum to one, so dV summed over keys is dO summed over the rows
    that see a key. dO = 0 gives zero gradients; rows without a key give dQ = 0."""
    for n, (Nq, Nkv, mode, W, G) in enumerate([(40, 40, 0, 0, 0), (40, 40, 1, 0, 0),
                                               (30, 50, 2, 7, 3), (50, 30, 3, 4, 0),
                                               (36, 36, 4, 0, 9)]):
        q = _rand((2, 2, Nq, 8), 4200 + n)
        k = _rand((2, 2, Nkv, 8), 4210 + n)
        v = _rand((2, 2, Nkv, 8), 4220 + n)
        g = _rand((2, 2, Nq, 8), 4230 + n)
        dq, dk, dv = orc.attention_backward(q, k, v, g, 0.4, mode, W, G)
        assert np.abs(dk.sum(axis=2)).max() < 1e-12, n
        seen = np.array([visible_count(i + Nkv - Nq, Nkv, mode, W, G) > 0 for i in range(Nq)])
        want = g.astype(np.float64)[:, :, seen].sum(axis=2)
        assert np.allclose(dv.sum(axis=2), want, rtol=1e-12, atol=1e-12), n
        assert np.all(dq[:, :, ~seen] == 0), n
        z = orc.attention_backward(q, k, v, np.zeros_like(g), 0.4, mode, W, G)
        assert all(np.all(x == 0) for x in z), n


def pin_backward_block_sparse(orc):
    """Block-sparse gradients: torch autograd in float64 through a softmax masked by the layout
    expanded with a Kronecker product (ragged edges, rows and keys that no tile reaches);
    central differences of the oracle's block-sparse forward on tiny inputs; an all-ones
    layout gives exactly the unmasked gradients; the softmax Jacobian's invariants."""
    cases = [(1, 2, 13, 17, 8, 4), (2, 1, 20, 12, 4, 5), (1, 3, 9, 9, 8, 3), (2, 2, 16, 16, 8, 8)]
    for n, (B, H, Nq, Nkv, d, blk) in enumerate(cases):
        q = _rand((B, H, Nq, d), 4300 + 4 * n)
        k = _rand((B, H, Nkv, d), 4301 + 4 * n)
        v = _rand((B, H, Nkv, d), 4302 + 4 * n)
        g = _rand((B, H, Nq, d), 4303 + 4 * n)
        lay = _random_layout(H, -(-Nq // blk), -(-Nkv // blk), 4304 + n, density=0.5)
        lay[0, -1, :] = 0  # a query block that sees nothing
        scale = float(np.float32(1 / math.sqrt(d)))
        got = orc.attention_backward_block_sparse(q, k, v, g, scale, lay, blk)
        want = library_backward(q, k, v, g, scale, block_mask(lay, blk, Nq, Nkv))
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert np.allclose(a, b, rtol=1e-11, atol=1e-12), (n, name, np.abs(a - b).max())
        # invariants: dK sums to zero over keys, dV sums to dO over the rows that see a key,
        # rows that see nothing get dQ = 0
        dq, dk, dv = got
        seen = np.stack([block_mask(lay, blk, Nq, Nkv)[h].numpy().any(axis=1) for h in range(H)])
        assert np.abs(dk.sum(axis=2)).max() < 1e-12, n
        want_v = np.stack([g.astype(np.float64)[:, h, seen[h]].sum(axis=1) for h in range(H)], 1)
        assert np.allclose(dv.sum(axis=2), want_v, rtol=1e-12, atol=1e-12), n
        assert all(np.all(dq[:, h, ~seen[h]] == 0) for h in range(H)), n
        ones = np.ones_like(lay)
        dense = orc.attention_backward(q, k, v, g, scale, 0)
        full = orc.attention_backward_block_sparse(q, k, v, g, scale, ones, blk)
        assert all(np.array_equal(a, b) for a, b in zip(dense, full)), n
    h = 2.0 ** -10
    rng = np.random.default_rng(4350)
    Nq, Nkv, d, blk = 6, 7, 2, 2
    q, k, v, g = (np.round(rng.standard_normal(sh) * 64) / 64
                  for sh in ((1, 2, Nq, d), (1, 2, Nkv, d), (1, 2, Nkv, d), (1, 2, Nq, d)))
    q, k, v, g = (x.astype(np.float32) for x in (q, k, v, g))
    lay = np.array([[[1, 0, 1, 0], [0, 1, 1, 0], [1, 1, 0, 1]],
                    [[0, 1, 0, 1], [1, 0, 0, 0], [0, 0, 1, 1]]], np.uint8)
    dq, dk, dv = orc.attention_backward_block_sparse(q, k, v, g, 0.5, lay, blk)

    def loss(qq, kk, vv):
        o, _ = orc.attention_block_sparse(qq, kk, vv, 0.5, lay, blk)
        return float((o * g.astype(np.float64)).sum())

    for which, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += np.float32(h)
            xm[idx] -= np.float32(h)
            args_p = [xp if w == which else y for w, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if w == which else y for w, y in (("q", q), ("k", k), ("v", v))]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-5, atol=2e-6), (which, np.abs(grad - num).max())


def pin_prefill_paged(orc):
    """Chunked prefill against a paged cache: each sequence's newest q_lens[s] tokens attend
    to its seq_lens[s] keys with bottom-right masks. Pinned to torch SDPA in float64 on the
    contiguous keys (gathered before paging) with tril masks of the chunk's shape; a
    different physical placement is bit-identical; a chunk of one token is single-token
    decode; a whole-sequence chunk is the contiguous causal case."""
    H, d, ps = 2, 8, 16
    lens = [1, 16, 17, 40, 64, 33]
    qls = [1, 5, 17, 12, 64, 0]
    Qmax = 64
    ks = [_rand((L, H, d), 4400 + i) for i, L in enumerate(lens)]
    vs = [_rand((L, H, d), 4410 + i) for i, L in enumerate(lens)]
    q = _rand((len(lens), Qmax, H, d), 4420)
    kp, vp, pt = make_paged(ks, vs, ps, 9)
    scale = float(np.float32(0.35))
    for mode, W, G in [(1, 0, 0), (0, 0, 0), (2, 5, 3), (3, 4, 0), (4, 0, 7)]:
        o, l = orc.prefill_paged(q, kp, vp, pt, np.array(lens, np.int32),
                                 np.array(qls, np.int32), 0.35, mode, W, G)
        for s, (L, nq) in enumerate(zip(lens, qls)):
            assert np.all(np.isnan(o[s, nq:])) and np.all(np.isnan(l[s, nq:])), s
            if nq == 0:
                continue
            qc = np.ascontiguousarray(q[s, :nq].transpose(1, 0, 2))[None]
            kc = np.ascontiguousarray(ks[s].transpose(1, 0, 2))[None]
            vc = np.ascontiguousarray(vs[s].transpose(1, 0, 2))[None]
            m = band_mask(nq, L, mode, W, G)
            ro, rl = library_attention_mask(qc, kc, vc, scale, m)
            fin = m.any(dim=1).numpy()
            got_o = o[s, :nq].transpose(1, 0, 2)
            got_l = l[s, :nq].transpose(1, 0)
            assert np.allclose(got_o[:, fin], ro[0][:, fin], rtol=1e-12, atol=1e-13), (mode, s)
            assert np.allclose(got_l[:, fin], rl[0][:, fin], rtol=1e-12, atol=1e-13), (mode, s)
            assert np.all(got_l[:, ~fin] == -np.inf) and np.all(got_o[:, ~fin] == 0), (mode, s)
        kp2, vp2, pt2 = make_paged(ks, vs, ps, 10, spare=4)
        o2, l2 = orc.prefill_paged(q, kp2, vp2, pt2, np.array(lens, np.int32),
                                   np.array(qls, np.int32), 0.35, mode, W, G)
        assert np.array_equal(o, o2, equal_nan=True) and np.array_equal(l, l2, equal_nan=True)
    # one-token chunks are decode (the newest token sees every key)
    ones = np.ones(len(lens), np.int32)
    o, l = orc.prefill_paged(q, kp, vp, pt, np.array(lens, np.int32), ones, 0.35, 1)
    do, dl = orc.decode_paged(np.ascontiguousarray(q[:, 0]), kp, vp, pt,
                              np.array(lens, np.int32), 0.35)
    assert np.array_equal(o[:, 0], do) and np.array_equal(l[:, 0], dl)


def multimodal_mask(n_img, n_txt):
    """The article's multimodal visibility written block by block: image->image all,
    image->text none, text->image all, text->text causal (tril)."""
    n = n_img + n_txt
    m = torch.zeros(n, n, dtype=torch.bool)
    m[:n_img, :n_img] = True
    m[n_img:, :n_img] = True
    m[n_img:, n_img:] = torch.tril(torch.ones(n_txt, n_txt, dtype=torch.bool))
    return m


def pin_merge_lse(orc):
    """Merging the results over two disjoint key sets (an arbitrary split, not contiguous)
    gives torch SDPA over their union; an empty side leaves the other unchanged; two empty
    sides give O = 0, LSE = -inf; the merge is symmetric."""
    q = _rand((2, 2, 11, 8), 4500) * 2
    k = _rand((2, 2, 37, 8), 4501) * 2
    v = _rand((2, 2, 37, 8), 4502)
    scale = float(np.float32(0.45))
    pick = torch.from_numpy(np.random.default_rng(4503).random(37) < 0.4)
    ma = pick[None, :].expand(11, 37).clone()
    mb = ~ma
    oa, la = library_attention_mask(q, k, v, scale, ma)
    ob, lb = library_attention_mask(q, k, v, scale, mb)
    ro, rl = library_attention_mask(q, k, v, scale, torch.ones(11, 37, dtype=torch.bool))
    # the merge reads float32 inputs; give it exactly representable values of the parts
    oa32, la32, ob32, lb32 = (np.asarray(x, np.float32) for x in (oa, la, ob, lb))
    o, l = orc.merge_lse(oa32, la32, ob32, lb32)
    # rounding the parts to float32 moves each lse by at most |lse| 2^-24 and each weight by
    # a relative 2 |lse| 2^-24, so the union is met to within a few of those
    eps = 4 * 2.0 ** -24 * max(np.abs(la).max(), np.abs(lb).max(), 1.0)
    assert np.abs(l - rl).max() <= eps
    assert np.abs(o - ro).max() <= 4 * eps * max(np.abs(ro).max(), 1.0)
    o2, l2 = orc.merge_lse(ob32, lb32, oa32, la32)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    ninf = np.full_like(la32, -np.inf)
    o3, l3 = orc.merge_lse(oa32, la32, np.zeros_like(ob32), ninf)
    assert np.array_equal(o3, oa32.astype(np.float64)) and np.array_equal(l3, la32)
    o4, l4 = orc.merge_lse(np.zeros_like(oa32), ninf, np.zeros_like(ob32), ninf)
    assert np.all(o4 == 0) and np.all(l4 == -np.inf)


def pin_multimodal(orc):
    """The multimodal oracle against torch SDPA with the block-by-block multimodal mask, and
    against the article's three-call split (image full, text causal, text to image)
    merged by log-sum-exp."""
    B, H, ni, nt, d = 1, 2, 9, 14, 8
    qi, ki, vi = (_rand((B, H, ni, d), 4600 + i) for i in range(3))
    qt, kt, vt = (_rand((B, H, nt, d), 4610 + i) for i in range(3))
    scale = float(np.float32(0.4))
    oi, li, ot, lt = orc.multimodal(qi, ki, vi, qt, kt, vt, scale)
    q = np.concatenate([qi, qt], 2)
    k = np.concatenate([ki, kt], 2)
    v = np.concatenate([vi, vt], 2)
    ro, rl = library_attention_mask(q, k, v, scale, multimodal_mask(ni, nt))
    assert np.allclose(oi, ro[:, :, :ni], rtol=1e-12, atol=1e-13)
    assert np.allclose(ot, ro[:, :, ni:], rtol=1e-12, atol=1e-13)
    assert np.allclose(li, rl[:, :, :ni], rtol=1e-12, atol=1e-13)
    assert np.allclose(lt, rl[:, :, ni:], rtol=1e-12, atol=1e-13)
    o1, l1 = library_attention_mask(qi, ki, vi, scale, torch.ones(ni, ni, dtype=torch.bool))
    o2, l2 = library_attention_mask(qt, kt, vt, scale, torch.tril(torch.ones(nt, nt,
                                                                             dtype=torch.bool)))
    o3, l3 = library_attention_mask(qt, ki, vi, scale, torch.ones(nt, ni, dtype=torch.bool))
    assert np.allclose(oi, o1, rtol=1e-12, atol=1e-13) and np.allclose(li, l1, rtol=1e-12)
    lm = np.logaddexp(l2, l3)
    om = np.exp(l2 - lm)[..., None] * o2 + np.exp(l3 - lm)[..., None] * o3
    assert np.allclose(ot, om, rtol=1e-12, atol=1e-13) and np.allclose(lt, lm, rtol=1e-12)


ALL_PINS = [pin_library, pin_mpmath, pin_q_zero, pin_causal_row0, pin_onehot_edges,
            pin_rows_sum_to_one, pin_shift, pin_permutation, pin_split_merge,
            pin_mask_reductions, pin_empty_rows, pin_decode, pin_library_more_masks,
            pin_mpmath_more_masks, pin_q_zero_more_masks, pin_onehot_more_edges,
            pin_more_mask_reductions, pin_backward_library, pin_backward_finite_difference,
            pin_backward_invariants, pin_backward_block_sparse, pin_prefill_paged,
            pin_merge_lse, pin_multimodal]
