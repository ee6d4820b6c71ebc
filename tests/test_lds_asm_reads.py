"""The GEMM kernels read LDS fragments with inline-assembly ds_read instructions that the
compiler does not track: it takes their result registers as written the moment the
instruction issues. If it then copies, spills or reuses such a register before the
kernel's own s_waitcnt lgkmcnt(0), the copy holds stale data, or the arriving data
overwrites another value (an address, say). This test compiles the kernel sources to
gfx950 assembly with the library's own flags and checks, in every straight run of code,
that no instruction other than another LDS read names a register of an inline-assembly
LDS read still in flight. (It reads the assembly of code built here from this
repository's sources only.)"""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from latent_moe_layer_sigmoid_amd import build_lib

SOURCES = ["gemm_tiled.hip", "gemm_mx.hip"]


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]", text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def in_flight_touches(asm_text):
    """{kernel symbol: [(line, instruction, register)]} for every instruction that names a
    register an inline-assembly LDS read writes, after the read and before an
    s_waitcnt lgkmcnt(0) in the same basic block."""
    found = {}
    for func in re.split(r"\n(?=\S+:\s*; @)", asm_text):
        name = func.split(":", 1)[0].strip()
        if not name.startswith("_Z"):
            continue
        pending, hits, inside = {}, [], False
        for i, line in enumerate(func.splitlines()):
            if ";;#ASMSTART" in line:
                inside = True
                continue
            if ";;#ASMEND" in line:
                inside = False
                continue
            s = line.split(";")[0].strip()
            if not s:
                continue
            op = s.split()[0]
            if s.endswith(":") or op.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
                pending = {}                    # block boundary: only straight runs are checked
                continue
            if op == "s_waitcnt":
                if "lgkmcnt(0)" in s:
                    pending = {}
                continue
            operands = s[len(op):]
            if op.startswith(("ds_read", "ds_load")):
                dst, _, src = operands.partition(",")
                hits += [(i, s, r) for r in _regs(src) if r in pending]
                if inside:
                    pending.update({r: i for r in _regs(dst)})
                continue
            hits += [(i, s, r) for r in _regs(operands) if r in pending]
        found[name] = hits
    return found


def _assemble(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [build_lib.hipcc(), *build_lib.FLAGS, "--cuda-device-only", "-S",
           os.path.join(build_lib.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return src, open(out).read()


def _have_hipcc():
    try:
        build_lib.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not found")
def test_inline_lds_read_registers_untouched_until_waited():
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
            listings = list(ex.map(lambda s: _assemble(s, d), SOURCES))
    n_kernels = 0
    for src, text in listings:
        assert ";;#ASMSTART" in text, f"{src}: no inline-assembly LDS reads left to check"
        for name, hits in in_flight_touches(text).items():
            n_kernels += 1
            assert not hits, f"{src} {name}: registers of an LDS read in flight touched: {hits[:4]}"
    assert n_kernels >= 5


def test_checker_finds_a_copy_of_a_register_in_flight():
    """The checker itself, on a hand-written listing: a copy out of a read's register
    before the wait is reported; the same copy after the wait, or in another block, is not."""
    listing = "\n".join([
        "_Zkernel:  ; @_Zkernel",
        "\t;;#ASMSTART",
        "\tds_read_b128 v[10:13], v2 offset:0",
        "\t;;#ASMEND",
        "\tv_mfma_f32_32x32x16_bf16 v[20:35], v[40:43], v[44:47], v[20:35]",
        "\tv_mov_b64_e32 v[50:51], v[12:13]",
        "\ts_waitcnt lgkmcnt(0)",
        "\tv_mov_b64_e32 v[52:53], v[12:13]",
        "\t;;#ASMSTART",
        "\tds_read_b128 v[14:17], v2 offset:0x200",
        "\t;;#ASMEND",
        ".LBB0_1:",
        "\tv_mov_b64_e32 v[54:55], v[14:15]",
        "\ts_endpgm",
    ])
    hits = in_flight_touches(listing)["_Zkernel"]
    assert sorted(r for _, _, r in hits) == [("v", 12), ("v", 13)]
    assert all(s == "v_mov_b64_e32 v[50:51], v[12:13]" for _, s, _ in hits)
