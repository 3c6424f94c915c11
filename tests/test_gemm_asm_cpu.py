"""Static check of the compiled direct-to-LDS kernels (no GPU needed).

The direct-to-LDS GEMM and the head_dim-128 attention dK/dV kernel issue LDS
reads as inline asm (the GEMM's transpose reads, every tile read of the
attention kernel), outside the compiler's wait tracking, and wait for them
themselves with s_waitcnt lgkmcnt(0).  This test compiles the sources to
gfx950 assembly with the library's own flags and walks every such kernel:
between an untracked LDS read and the next lgkmcnt(0) wait, no instruction
may read or overwrite the read's destination registers, and no branch or
label may intervene (the result lands asynchronously, so an early use would
see stale data)."""
import os
import re
import subprocess
import tempfile

import pytest

from layer_streamed_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for a, b, c in _REG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _device_asm(src):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in build.HIP_FLAGS if f != "-fPIC"]
        subprocess.run([build.HIPCC] + flags + ["--cuda-device-only", "-S",
                                                os.path.join(CSRC, src), "-o", out],
                       check=True, capture_output=True)
        return open(out).read()


def _kernels(asm, pattern):
    """(name, body lines) of every kernel whose symbol contains `pattern`."""
    ks = []
    cur, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*" + pattern + r"\S*):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is not None:
            if "s_endpgm" in line:
                ks.append((cur, body))
                cur = None
            else:
                body.append(line)
    return ks


def _check(body):
    pending = set()
    in_asm = False
    for line in body:
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if not code or code.startswith("."):
            if code.startswith(".LBB") and pending:
                return f"label with transpose reads in flight: {code}"
            continue
        op = code.split()[0]
        if op == "s_waitcnt" and "lgkmcnt(0)" in code:
            pending.clear()
            continue
        if op.startswith("s_cbranch") or op == "s_branch" or op == "s_setpc_b64":
            if pending:
                return f"branch with transpose reads in flight: {code}"
            continue
        if op == "ds_read_b64_tr_b16" or (in_asm and op.startswith("ds_read")):
            dst, addr = code[len(op):].split(",", 1)
            if _regs(addr) & pending or _regs(dst) & pending:
                return f"transpose read uses an in-flight register: {code}"
            pending |= _regs(dst)
            continue
        if _regs(code[len(op):]) & pending:
            return f"in-flight transpose result touched: {code}"
    return None if not pending else "kernel ends with transpose reads in flight"


@pytest.mark.parametrize("src,pattern", [("gemm.hip", "gemm_dl_kernel"),
                                         ("attention.hip", "attn_dkdv_dl_kernel")])
def test_untracked_lds_reads_are_waited_for_before_use(src, pattern):
    kernels = _kernels(_device_asm(src), pattern)
    with_tr = [(n, b) for n, b in kernels if any("ds_read_b64_tr_b16" in l for l in b)]
    assert with_tr, f"no {pattern} kernel with transpose reads found"
    bad = {n: e for n, b in with_tr if (e := _check(b))}
    assert not bad, bad


def test_checker_catches_planted_early_use():
    ok = ["ds_read_b64_tr_b16 v[10:11], v5", "ds_read_b64_tr_b16 v[12:13], v6",
          "s_waitcnt lgkmcnt(0)", "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert _check(ok) is None
    early = ["ds_read_b64_tr_b16 v[10:11], v5", "v_mov_b32_e32 v30, v11", "s_waitcnt lgkmcnt(0)"]
    assert "touched" in _check(early)
    clobber = ["ds_read_b64_tr_b16 v[10:11], v5", "v_add_u32_e32 v10, 4, v7", "s_waitcnt lgkmcnt(0)"]
    assert "touched" in _check(clobber)
    partial = ["ds_read_b64_tr_b16 v[10:11], v5", "s_waitcnt lgkmcnt(1)",
               "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert "touched" in _check(partial)
    branch = ["ds_read_b64_tr_b16 v[10:11], v5", "s_cbranch_scc1 .LBB0_3"]
    assert "branch" in _check(branch)
    # an asm-issued row read is untracked too; a compiler-issued one is not
    asm_row = [";;#ASMSTART", "ds_read_b128 v[10:13], v5", ";;#ASMEND",
               "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert "touched" in _check(asm_row)
    compiler_row = ["ds_read_b128 v[10:13], v5",
                    "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert _check(compiler_row) is None
