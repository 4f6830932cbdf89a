"""The direct-to-LDS copies are inline asm that set M0 (the LDS destination of
global_load_lds_*) and list it as clobbered.  The compiler treats M0 as reserved and
does not keep its own values across such a clobber, so the kernels are correct only
while nothing the compiler emits uses M0.  This test compiles every kernel source
with the library's own flags to gfx950 assembly and checks exactly that: every
mention of M0 is the asm's `s_mov_b32 m0, <sgpr>` directly followed by `s_nop 0` and
a `global_load_lds_*`, every `global_load_lds_*` follows such a write, and no
instruction that reads M0 implicitly (indexed register moves, messages, GWS, ordered
counts, interpolation, buffer loads into LDS) appears.  CPU only: it compiles and
reads text, nothing runs."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fine_grained_block_token_amd import _build

KERNEL_SOURCES = ["cast.hip", "gemm.hip", "gemm_wide.hip"]
IMPLICIT_M0 = ("v_movrel", "s_movrel", "s_sendmsg", "ds_gws", "ds_ordered_count", "v_interp", "s_set_gpr_idx",
               "ds_param_load", "ds_direct_load", "lds_param_load", "lds_direct_load")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _assembly(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [HIPCC, *_build.flags_for(src), "-I", os.path.join(_build.ROOT, "include"), "-I", _build.CSRC,
           "--cuda-device-only", "-S", os.path.join(_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return src, open(out).read()


def _instructions(text):
    ins = []
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        ins.append(s)
    return ins


@pytest.fixture(scope="module")
def kernel_assembly(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
        return dict(ex.map(lambda s: _assembly(s, d), KERNEL_SOURCES))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_m0_is_only_the_copy_destination(kernel_assembly, src):
    ins = _instructions(kernel_assembly[src])
    copies = 0
    for i, s in enumerate(ins):
        op = s.split()[0]
        assert not op.startswith(IMPLICIT_M0), f"{src}: implicit M0 user: {s}"
        assert not (op.startswith("buffer_") and re.search(r"\blds\b", s)), f"{src}: buffer load into LDS: {s}"
        if re.search(r"\bm0\b", s):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", s), f"{src}: M0 used outside the copy asm: {s}"
            assert ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_dword"), \
                f"{src}: M0 write not followed by its copy: {ins[i:i + 3]}"
        if op.startswith("global_load_lds_dword"):
            copies += 1
            assert i >= 2 and re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 2]) and ins[i - 1] == "s_nop 0", \
                f"{src}: copy without its own M0 write: {ins[max(0, i - 2):i + 1]}"
    # the GEMMs stage every tile through these copies; the casts use none
    assert (copies > 0) == src.startswith("gemm"), (src, copies)
