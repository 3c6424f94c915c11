"""Static check of the compiled direct-to-LDS kernels (no GPU needed).

The direct-to-LDS GEMM and the head_dim-128 attention dK/dV kernel issue LDS
reads as inline asm (the GEMM's transpose reads, every tile read of the
attention kernel), outside the compiler's wait tracking, and wait for them
themselves with s_waitcnt lgkmcnt.  This test compiles the sources to
gfx950 assembly with the library's own flags and walks every such kernel:
between an untracked LDS read and the wait that retires it, no instruction
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
        flags = [f for f in build.hip_flags(src) if f != "-fPIC"]
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


_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def _check(body):
    # outstanding LDS/scalar-memory operations, oldest first: the register set
    # of an untracked read, or None for one the compiler issued.  LDS returns
    # in order, so lgkmcnt(N) retires all but the N newest; a scalar or flat
    # load may return out of order, and while one is outstanding only
    # lgkmcnt(0) retires anything.
    pending = []
    in_asm = False

    def live():
        out = set()
        for _, regs in pending:
            out |= regs or set()
        return out

    for line in body:
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if not code or code.startswith("."):
            if code.startswith(".LBB") and live():
                return f"label with transpose reads in flight: {code}"
            continue
        op = code.split()[0]
        if op == "s_waitcnt":
            m = _LGKM.search(code)
            if m:
                n = int(m.group(1))
                if n == 0:
                    pending.clear()
                elif not any(kind == "unordered" for kind, _ in pending):
                    del pending[:max(0, len(pending) - n)]
            continue
        if op.startswith("s_cbranch") or op == "s_branch" or op == "s_setpc_b64":
            if live():
                return f"branch with transpose reads in flight: {code}"
            continue
        if op == "ds_read_b64_tr_b16" or (in_asm and op.startswith("ds_read")):
            dst, addr = code[len(op):].split(",", 1)
            if _regs(addr) & live() or _regs(dst) & live():
                return f"transpose read uses an in-flight register: {code}"
            pending.append(("lds", _regs(dst)))
            continue
        if _regs(code[len(op):]) & live():
            return f"in-flight transpose result touched: {code}"
        if op.startswith("ds_"):
            pending.append(("lds", None))
        elif op.startswith(("s_load", "s_buffer_load", "flat_", "s_memtime", "s_memrealtime")):
            pending.append(("unordered", None))
    return None if not live() else "kernel ends with transpose reads in flight"


@pytest.mark.parametrize("src,pattern", [("gemm.hip", "gemm_dl_kernel"),
                                         ("attention.hip", "attn_dkdv_dl_kernel"),
                                         ("attention.hip", "attn_dq_dl_kernel"),
                                         ("attention.hip", "attn_fwd_dl_kernel")])
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
    # lgkmcnt(N) retires all but the N newest reads
    pipelined = ["ds_read_b64_tr_b16 v[10:11], v5", "ds_read_b64_tr_b16 v[12:13], v6",
                 "ds_read_b64_tr_b16 v[14:15], v7", "s_waitcnt lgkmcnt(1)",
                 "v_mfma_f32_16x16x32_bf16 v[0:3], v[10:13], v[20:23], v[0:3]",
                 "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v30, v15"]
    assert _check(pipelined) is None
    too_new = ["ds_read_b64_tr_b16 v[10:11], v5", "ds_read_b64_tr_b16 v[12:13], v6",
               "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v30, v12", "s_waitcnt lgkmcnt(0)"]
    assert "touched" in _check(too_new)
    # a compiler LDS op issued after the read counts too
    counted = ["ds_read_b64_tr_b16 v[10:11], v5", "ds_read_b32 v40, v6",
               "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v30, v10"]
    assert _check(counted) is None
    # a scalar load may return out of order: only lgkmcnt(0) retires then
    scalar = ["ds_read_b64_tr_b16 v[10:11], v5", "s_load_dword s4, s[0:1], 0x0",
              "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v30, v10"]
    assert "touched" in _check(scalar)
    branch = ["ds_read_b64_tr_b16 v[10:11], v5", "s_cbranch_scc1 .LBB0_3"]
    assert "branch" in _check(branch)
    # an asm-issued row read is untracked too; a compiler-issued one is not
    asm_row = [";;#ASMSTART", "ds_read_b128 v[10:13], v5", ";;#ASMEND",
               "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert "touched" in _check(asm_row)
    compiler_row = ["ds_read_b128 v[10:13], v5",
                    "v_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]"]
    assert _check(compiler_row) is None
