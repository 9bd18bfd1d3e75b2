"""Invariants of the compiled kernels that their sources rely on.

The image prefetch of the forward and reverse round kernels and the tile
copies of tree attention are issued in inline assembly that writes M0
(csrc/chunk.h, lds_load16_untracked).  M0 is a reserved register: a clobber
list cannot protect it, so these kernels must keep nothing else in it.  This
test compiles the kernel sources for gfx950 and checks, in their AMD
assembly, that every access to M0 is one of those copies (a write
immediately followed by the wait state and the load), and that no indirect
register indexing (which reads M0) appears.
CPU only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_packed_chunkwise_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-O3", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}", "--cuda-device-only", "-S",
           src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
@pytest.mark.parametrize("name", ["kda_fwd.hip", "kda_bwd.hip", "attn.hip"])
def test_m0_only_in_the_image_copies(name, tmp_path):
    lines = [l.strip() for l in _asm(os.path.join(CSRC, name), tmp_path)]
    code = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    n_copy = 0
    for i, l in enumerate(code):
        assert not l.startswith(("s_movrel", "v_movrel", "s_set_gpr_idx")), l
        if re.search(r"\bm0\b", l) is None:
            continue
        if l.startswith("s_mov_b32 m0,"):
            assert code[i + 1] == "s_nop 0", (l, code[i + 1])
            assert code[i + 2].startswith("global_load_lds_dwordx4"), (l, code[i + 2])
            n_copy += 1
        else:
            pytest.fail(f"{name}: M0 used outside the image copies: {l}")
    assert n_copy > 0
