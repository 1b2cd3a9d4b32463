"""Plausible mistakes planted in a copy of the oracle source (for sensitivity tests).

Each entry replaces one unique snippet of oracle/attention.c. The copy is built with gcc on
the CPU into a temporary library; the real oracle is never modified.
"""
import oracle
from oracle import build as obuild

MUTANTS = {
    "causal_strict": ("return j <= ip;", "return j < ip;"),
    "window_inclusive": ("(ip - j) < window", "(ip - j) <= window"),
    "global_inclusive": ("j < n_global", "j <= n_global"),
    "window_not_causal": ("return j <= ip && ((ip - j)", "return j <= ip + 1 && ((ip - j)"),
    "no_max_subtraction": ("e = exp(s[j] - m);", "e = exp(s[j]);"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "value_as_key": ("(double)krow[j][c];", "(double)vrow[j][c];"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "query_index": ("dot += (double)q[c]", "dot += (double)q[0]"),
    "no_normalise": ("out[c] /= l;", "out[c] /= (l + 1.0);"),
    "top_left_causal": ("i + (Nkv - Nq), mode", "i, mode"),
    "page_slot": ("(size_t)(j % page_size)", "(size_t)((j + 1) % page_size)"),
    "decode_head": ("* H + h) * d;", "* H + 0) * d;"),
    "max_ignores_first": ("if (s[j] > m)", "if (j > 0 && s[j] > m)"),
    "band_narrow_left": ("j >= ip - window &&", "j > ip - window &&"),
    "band_wide_right": ("j <= ip + window;", "j <= ip + window + 1;"),
    "prefix_inclusive": ("j < prefix ||", "j <= prefix ||"),
    "prefix_not_causal": ("j - ip <= 0;", "j - ip <= 1;"),
    "block_query_index": ("(size_t)(i / block)) * nkb", "(size_t)((i + 1) / block)) * nkb"),
    "block_key_index": ("lrow[j / block] != 0", "lrow[(j + 1) / block] != 0"),
    "block_head": ("long h = bh % H;", "long h = 0;"),
    "bwd_no_rowterm": ("ds = p[j] * (dp - D);", "ds = p[j] * dp;"),
    "bwd_block_key_index": ("lrow[j / block] == 0", "lrow[(j + 1) / block] == 0"),
    "bwd_block_query_index": ("(size_t)i / (size_t)block) * nkb",
                              "(size_t)(i + 1) / (size_t)block) * nkb"),
    "bwd_block_head": ("layout + ((size_t)(bh % H) * nqb", "layout + ((size_t)(bh / H) * nqb"),
    "bwd_dk_no_scale": ("dkb[(size_t)j * d + c] += scale * ds", "dkb[(size_t)j * d + c] += ds"),
    "bwd_dv_from_ds": ("dvb[(size_t)j * d + c] += p[j] * (double)gi[c];",
                       "dvb[(size_t)j * d + c] += ds * (double)gi[c];"),
    "bwd_rowterm_from_v": ("D += (double)gi[c] * orow[c];",
                           "D += (double)gi[c] * (double)vb[c];"),
    "bwd_dq_uses_q": ("scale * ds * (double)kb[(size_t)j * d + c];",
                      "scale * ds * (double)qi[c];"),
    "prefill_top_left": ("i + (L - nq), mode", "i, mode"),
    "prefill_row_stride": ("((size_t)sq * Qmax + (size_t)i) * H + (size_t)h;",
                           "((size_t)sq * Qmax + (size_t)i) * H;"),
    "prefill_page_slot": ("slot = j - pg * page_size;", "slot = (j + 1) % page_size;"),
    "prefill_value_head": ("vp[j] = v_pages + (tok * (size_t)H + (size_t)h)",
                           "vp[j] = v_pages + (tok * (size_t)H + (size_t)0)"),
    "prefill_chunk_shift": ("i + (L - nq), mode", "i + (L - nq) - 1, mode"),
    "merge_weight_swap": ("wa = exp(la - m);", "wa = exp(lb - m);"),
    "merge_lse_no_max": ("lse[r] = m + log(t);", "lse[r] = log(t);"),
    "merge_not_normalised": ("o_b[(size_t)r * d + c]) / t;", "o_b[(size_t)r * d + c]);"),
}


def build_mutant(name, tmpdir):
    before, after = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique"
    path = f"{tmpdir}/mutant_{name}.c"
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    lib = obuild.build(path, f"{tmpdir}/libmutant_{name}.so")
    return oracle.Oracle(lib)
