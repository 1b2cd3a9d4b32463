"""Static checks of the dK/dV kernel's hand-placed hazard padding, on the gfx950 assembly that
hipcc makes of the backward's source (CPU only; no GPU needed).

The dK/dV kernel accumulates dK and dV in the AGPR file through inline-asm MFMAs, which the
compiler's hazard recognizer does not see. The source covers the two hazards itself:
  * a vector write of an MFMA operand needs wait states before the MFMA reads it: every
    inline MFMA carries an `s_nop 2` in front of it;
  * an MFMA's result must be complete before other instructions read it (up to 18 wait
    states for 16 passes): the accumulators go through padding of 24 wait states after the
    loop, in statements that take them as operands.
These tests read the file's assembly (compiled with the library's flags,
conftest.device_asm) and check, in every dK/dV instantiation, that the padding is where the
source means it to be: before every AGPR-accumulating MFMA, between the last of them and the
first instruction that reads an accumulator, and that the loop holds no copies between the
register files. The compiler may also copy an accumulator on its own (a move between AGPRs
when it splits a live range); placed right after an inline MFMA, such a copy reads the
register before the MFMA has written it, so every instruction that reads an AGPR is checked
against the last MFMA that writes it, in program order.
"""
import re

import pytest

MIN_WAIT_STATES = 19


@pytest.fixture(scope="module")
def asm(device_asm):
    return device_asm["fa_bwd.hip"]


def kernels(lines):
    """(name, instruction lines) of every dK/dV kernel in the file."""
    out = []
    for i, ln in enumerate(lines):
        if ln.startswith("_ZN") and "bwd_dkdv_kernel" in ln and ln.split(";")[0].rstrip().endswith(":"):
            j = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
            body = []
            for t in lines[i + 1:j]:
                t = t.split(";")[0].strip()
                if t and not t.startswith(".") and not t.endswith(":"):
                    body.append(t)
            out.append((ln.split(":")[0], body))
    return out


def loops(lines, name):
    """Instruction lists of the innermost loops (a label up to a branch back to it, holding no
    other such span and no s_endpgm) of kernel `name`."""
    i = next(k for k, ln in enumerate(lines) if ln.startswith(name + ":"))
    j = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
    seq, at = [], {}
    for t in lines[i + 1:j]:
        t = t.split(";")[0].strip()
        if re.match(r"\.LBB\w+:$", t):
            at[t[:-1]] = len(seq)
        elif t and not t.startswith("."):
            seq.append(t)
    spans = []
    for k, t in enumerate(seq):
        m = re.match(r"s_c?branch\w*\s+(\.LBB\w+)$", t)
        if m and m.group(1) in at and at[m.group(1)] <= k:
            a = at[m.group(1)]
            # a backward jump over the program's end is a block placed after it (e.g. one arm
            # of a branch jumping back to the join), not a loop
            if not any(x.startswith("s_endpgm") for x in seq[a:k + 1]):
                spans.append((a, k))
    return [seq[a:k + 1] for a, k in spans] if not spans else [
        seq[a:k + 1] for a, k in spans
        if not any((a2, k2) != (a, k) and a <= a2 and k2 <= k for a2, k2 in spans)]


def agprs(operand):
    """AGPR indices named by one operand (a5, a[0:15]); empty for anything else."""
    m = re.fullmatch(r"a(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"a\[(\d+):(\d+)\]", operand)
    return set(range(int(m.group(1)), int(m.group(2)) + 1)) if m else set()


def is_agpr_mfma(t):
    return re.match(r"v_mfma\S*\s+a\[", t) is not None


def wait_states(t):
    m = re.match(r"s_nop\s+(\d+)", t)
    return int(m.group(1)) + 1 if m else 1


def reads_agpr(t):
    """An instruction other than an MFMA that reads an AGPR (a source operand a<n> or a[..])."""
    if t.startswith("v_mfma"):
        return False
    ops = t.split(None, 1)
    if len(ops) < 2:
        return False
    if ops[0].startswith("v_accvgpr_read"):
        return True
    srcs = [s.strip() for s in ops[1].split(",")]
    if ops[0].startswith(("global_store", "buffer_store", "ds_write", "flat_store", "scratch_store")):
        return any(re.match(r"a(\d+|\[)", s) for s in srcs)
    return any(re.match(r"a(\d+|\[)", s) for s in srcs[1:])


def test_every_dkdv_instantiation_found(asm):
    names = [n for n, _ in kernels(asm)]
    # bf16 and fp16, d 64 and 128, masks 0-4 and the block-sparse layout
    assert len(names) == 2 * 2 * 6, names


def test_operand_padding_before_each_inline_mfma(asm):
    for name, body in kernels(asm):
        n = 0
        for i, t in enumerate(body):
            if is_agpr_mfma(t):
                n += 1
                prev = body[i - 1]
                m = re.match(r"s_nop\s+(\d+)", prev)
                assert m and int(m.group(1)) >= 2, f"{name}: {t!r} after {prev!r}"
        assert n > 0, f"{name}: no AGPR-accumulating MFMA"


def test_results_settled_before_reads(asm):
    for name, body in kernels(asm):
        mf = [i for i, t in enumerate(body) if is_agpr_mfma(t)]
        last = mf[-1]
        first_read = next(i for i in range(last + 1, len(body)) if reads_agpr(body[i]))
        ws = sum(wait_states(t) for t in body[last + 1:first_read])
        assert ws >= MIN_WAIT_STATES, f"{name}: {ws} wait states before {body[first_read]!r}"


def test_no_register_file_copies_in_the_loop(asm):
    for name, _ in kernels(asm):
        hot = [lp for lp in loops(asm, name) if any(is_agpr_mfma(t) for t in lp)]
        assert hot, f"{name}: no loop with AGPR-accumulating MFMAs"
        for lp in hot:
            copies = [t for t in lp if t.startswith(("v_accvgpr_read", "v_accvgpr_write",
                                                     "v_accvgpr_mov"))]
            assert not copies, f"{name}: {len(copies)} AGPR copies in a loop, e.g. {copies[:3]}"


def agpr_sources(t):
    """AGPRs that a non-MFMA instruction reads."""
    ops = t.split(None, 1)
    if len(ops) < 2 or ops[0].startswith("v_mfma"):
        return set()
    srcs = [x.strip() for x in ops[1].split(",")]
    if not ops[0].startswith(("global_store", "buffer_store", "ds_write", "flat_store",
                              "scratch_store")):
        srcs = srcs[1:]
    return set().union(*(agprs(x) for x in srcs))


def test_every_accumulator_read_waits_for_its_mfma(asm):
    for name, body in kernels(asm):
        written = {}  # AGPR -> index of the last inline MFMA that writes it
        for i, t in enumerate(body):
            if is_agpr_mfma(t):
                for r in agprs(t.split(None, 1)[1].split(",")[0].strip()):
                    written[r] = i
                continue
            for r in agpr_sources(t):
                if r in written:
                    ws = sum(wait_states(x) for x in body[written[r] + 1:i])
                    assert ws >= MIN_WAIT_STATES, (
                        f"{name}: {t!r} reads a{r} {ws} wait states after {body[written[r]]!r}")
