"""Every kernel of the library compiles without scratch memory (CPU only; no GPU needed).

A kernel that spills vector registers to scratch, or keeps an array in private memory, still
computes the right result, so the parity tests cannot see it; it shows only as a slower kernel.
These tests read the code-object metadata of every kernel in the gfx950 assembly of each HIP
source (compiled with the library's flags, conftest.device_asm) and require no vector-register
spills and no private segment. Scalar-register spills are allowed: they go to lanes of a vector
register, not to memory (some forward instantiations with the window, band and prefix masks
have them, outside the steady loops).
"""
import re

import pytest

from tiled_exact_attention_forward_amd import build as b

HIP = [s for s in b.SOURCES if s.endswith(".hip")]


def kernel_metadata(lines):
    """{kernel name: {field: value}} from the amdhsa.kernels metadata block."""
    text = "\n".join(lines)
    meta = text[text.index("amdhsa.kernels:"):text.index(".end_amdgpu_metadata")]
    out = {}
    for entry in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry)
        if not name:
            continue
        out[name.group(1)] = {f: int(v) for f, v in
                              re.findall(r"\.(\w+):\s+(\d+)\s*$", entry, flags=re.M)}
    return out


@pytest.mark.parametrize("src", HIP)
def test_no_scratch(device_asm, src):
    meta = kernel_metadata(device_asm[src])
    assert meta, f"{src}: no kernels found"
    for name, m in meta.items():
        assert m["vgpr_spill_count"] == 0, f"{src}: {name} spills {m['vgpr_spill_count']} VGPRs"
        assert m["private_segment_fixed_size"] == 0, (
            f"{src}: {name} uses {m['private_segment_fixed_size']} bytes of private memory")


def test_every_source_has_its_kernels(device_asm):
    counts = {s: len(kernel_metadata(device_asm[s])) for s in HIP}
    # forward 60 (two dtypes, two head dims, masks, dense/paged/two-part and fp32), backward
    # 48, fp32 backward 24, decode 14, merge 6
    assert counts == {"fa_fwd.hip": 60, "fa_bwd.hip": 48, "fa_bwd32.hip": 24,
                      "fa_decode.hip": 14, "fa_merge.hip": 6}, counts
