import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def device_asm(tmp_path_factory):
    """gfx950 assembly of every HIP source of the library, compiled with the library's own
    flags (in parallel, once per session): {source file name: assembly lines}."""
    from tiled_exact_attention_forward_amd import build as b
    out_dir = tmp_path_factory.mktemp("device_asm")
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]

    def compile_one(src):
        out = out_dir / (src + ".s")
        cmd = ["hipcc", *b.FLAGS, *b.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(b.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}: {r.stderr[-3000:]}"
        return src, out.read_text().split("\n")

    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        return dict(ex.map(compile_one, srcs))
