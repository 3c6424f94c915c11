"""Static check of the compiled GEMM kernels (no GPU needed).

The direct-to-LDS GEMM issues its LDS transpose reads (ds_read_b64_tr_b16)
as inline asm, outside the compiler's wait tracking, and waits for them
itself with s_waitcnt lgkmcnt(0).  This test compiles gemm.hip to gfx950
assembly with the library's own flags and walks every such kernel: between
a transpose read and the next lgkmcnt(0) wait, no instruction may read or
overwrite the read's destination registers, and no branch or label may
intervene (the result lands asynchronously, so an early use would see stale
data)."""
import os
import re
import subprocess
import tempfile

import pytest

from layer_streamed_amd import build

SRC = os.path.join(os.path.dirname(build.__file__), "csrc", "gemm.hip")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for a, b, c in _REG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _device_asm():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        flags = [f for f in build.HIP_FLAGS if f != "-fPIC"]
        subprocess.run([build.HIPCC] + flags + ["--cuda-device-only", "-S", SRC, "-o", out],
                       check=True, capture_output=True)
        return open(out).read()


def _kernels(asm):
    """(name, body lines) of every direct-to-LDS GEMM kernel."""
    ks = []
    cur, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*gemm_dl_kernel\S*):", line)
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
    for line in body:
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
        if op == "ds_read_b64_tr_b16":
            dst, addr = code[len(op):].split(",", 1)
            if _regs(addr) & pending or _regs(dst) & pending:
                return f"transpose read uses an in-flight register: {code}"
            pending |= _regs(dst)
            continue
        if _regs(code[len(op):]) & pending:
            return f"in-flight transpose result touched: {code}"
    return None if not pending else "kernel ends with transpose reads in flight"


def test_transpose_reads_are_waited_for_before_use():
    kernels = _kernels(_device_asm())
    with_tr = [(n, b) for n, b in kernels if any("ds_read_b64_tr_b16" in l for l in b)]
    assert with_tr, "no direct-to-LDS kernel with transpose reads found"
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
