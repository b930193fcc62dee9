"""Checks on the gfx950 code the compiler generates for the HIP sources (host
only: hipcc cross-compiles, nothing runs on a GPU).

* No attention kernel (nor any other kernel outside the token selector) spills
  to scratch memory: the attention loaders may count their own vector-memory
  operations with a nonzero s_waitcnt vmcnt, and a scratch reload would add
  loads they do not count (and the compiler's waits for it would drain their
  copies in flight). The token selector's compute wavefronts issue no copies
  and its loader wavefronts wait for all their copies (vmcnt(0)) before
  publishing, so a spill there costs time only; its source is checked to hold
  no counted wait.
* M0 is touched only by the direct-to-LDS copy helpers: the compiler is not
  told that their inline asm writes M0 (a reserved register), so no compiler-
  generated instruction may keep a value in M0. Every instruction that names
  M0 must be the helper's own `s_mov_b32 m0, sN; s_nop 0;
  global_load_lds_dwordx4` sequence, and no other instruction that reads M0
  implicitly (relative moves, messages, GWS, LDS-DMA forms) may appear.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_attention_candidates_amd import build

pytestmark = pytest.mark.slow

HIPCC = build.HIPCC if os.path.exists(build.HIPCC) else shutil.which("hipcc")
HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
DMA_USERS = {"attention.hip", "token_select.hip"}
# mnemonics that read M0 without naming it
IMPLICIT_M0 = re.compile(r"(v_movrel|s_movrel|s_sendmsg|ds_gws|ds_ordered_count|v_interp|ds_\w*addtid|"
                         r"buffer_load_\w*lds|buffer_store_lds|global_load_lds)")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")

    def one(src):
        dst = out / (os.path.splitext(src)[0] + ".s")
        cmd = [HIPCC, *build.COMMON, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(build.PKG, "csrc", src), "-o", str(dst)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        return src, dst.read_text()

    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(one, HIP_SOURCES))


def _kernels(asm):
    """(name, private_segment_fixed_size) of every kernel in the metadata."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", asm, re.M)
    scratch = [int(x) for x in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", asm, re.M)]
    assert names and len(names) == len(scratch)
    return list(zip(names, scratch))


def _instructions(asm):
    """Instruction lines (no labels, directives or comments)."""
    out = []
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        out.append(s)
    return out


# sources whose ring waits are all vmcnt(0), so that scratch use is harmless
UNCOUNTED_WAITS = {"token_select.hip"}


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch(device_asm, src):
    if src in UNCOUNTED_WAITS:
        text = open(os.path.join(build.PKG, "csrc", src)).read()
        waits = re.findall(r"wait_vmcnt<([^>]*)>", text)
        assert waits and all(w.strip() == "0" for w in waits), f"{src}: counted vmcnt waits {waits}"
        return
    spilling = [n for n, size in _kernels(device_asm[src]) if size != 0]
    assert not spilling, f"{src}: kernels using scratch: {spilling}"


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_m0_only_in_lds_copies(device_asm, src):
    ins = _instructions(device_asm[src])
    uses = [i for i, s in enumerate(ins) if re.search(r"\bm0\b", s)]
    implicit = [i for i, s in enumerate(ins) if IMPLICIT_M0.match(s)]
    if src not in DMA_USERS:
        assert not uses and not implicit, f"{src}: unexpected M0 use: {ins[(uses + implicit)[0]]}"
        return
    assert uses, f"{src}: no direct-to-LDS copies found"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i]), f"{src}: compiler-generated M0 use: {ins[i]}"
        assert ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_dwordx4"), ins[i:i + 3]
    assert sorted(implicit) == sorted(i + 2 for i in uses), f"{src}: M0 reader outside the copy helpers"
