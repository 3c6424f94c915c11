"""Static checks of the compiled direct-to-LDS kernels (no GPU needed).

The direct-to-LDS GEMM and the head_dim-128 attention kernels stream their
operand tiles with global -> LDS copies issued as inline asm (an instruction
with no register result), so that the compiler's wait insertion does not
track them; every LDS read is an ordinary load or a compiler builtin, whose
waits the compiler places itself.  Two properties follow and are checked on
gfx950 assembly built with the library's own flags:

* no inline asm in any kernel issues a load that returns into registers (an
  asm load's destination is taken as written at once by the compiler, which
  may then reuse or copy those registers while the load is in flight);
* the compiler emits no vmcnt wait where copies may be in flight: inside a
  copy loop such a wait would also drain the copies of the next stage and
  serialize the ring (the kernels' own waits are asm, and each kernel
  retires its last copies with one before any code that follows its loop)."""
import os
import re
import subprocess
import tempfile

import pytest

from layer_streamed_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")
HIP_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


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


_ASM = {}


def _asm(src):
    if src not in _ASM:
        _ASM[src] = _device_asm(src)
    return _ASM[src]


def _kernels(asm, pattern=""):
    """(name, body lines) of every kernel whose symbol contains `pattern`."""
    ks = []
    cur, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*" + pattern + r"\S*):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is not None:
            if line.startswith(".Lfunc_end"):
                ks.append((cur, body))
                cur = None
            else:
                body.append(line)
    return ks


def _lines(body):
    """(in_asm, code) per instruction or label line, comments stripped."""
    out, in_asm = [], False
    for line in body:
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if code:
            out.append((in_asm, code))
    return out


_LOAD_WITH_RESULT = re.compile(r"^(ds_read|ds_load|global_load|buffer_load|flat_load|scratch_load|global_atomic|"
                               r"buffer_atomic|flat_atomic|ds_bpermute|ds_permute|ds_swizzle)")


def _asm_loads_with_result(body):
    bad = []
    for in_asm, code in _lines(body):
        if not in_asm:
            continue
        op = code.split()[0]
        if not _LOAD_WITH_RESULT.match(op):
            continue
        if op.startswith("global_load_lds") or (op.startswith("buffer_load") and " lds" in code):
            continue  # writes LDS only
        bad.append(code)
    return bad


def _drains_of_copies(body):
    """Compiler vmcnt waits that some path reaches while asm copies may be in
    flight: a may-analysis over the kernel's control-flow graph (blocks split
    at labels and branches), set by a copy, cleared by an asm vmcnt(0)."""
    lines = _lines(body)
    blocks, cur = [], []
    for in_asm, code in lines:
        if code.startswith(".LBB") and code.endswith(":"):
            if cur:
                blocks.append(cur)
            cur = [(in_asm, code)]
            continue
        cur.append((in_asm, code))
        op = code.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm"):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    where = {b[0][1][:-1]: i for i, b in enumerate(blocks) if b[0][1].startswith(".LBB")}

    def succ(i):
        last = blocks[i][-1][1]
        op = last.split()[0]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [where[last.split()[-1]]]
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if op.startswith("s_cbranch"):
            return nxt + [where[last.split()[-1]]]
        return nxt

    def run(i, state, bad=None):
        for in_asm, code in blocks[i]:
            op = code.split()[0]
            if in_asm and op.startswith("global_load_lds"):
                state = True
            elif op == "s_waitcnt" and "vmcnt" in code:
                if in_asm:
                    if "vmcnt(0)" in code:
                        state = False
                elif state and bad is not None:
                    bad.append(code)
        return state

    entry = [False] * len(blocks)
    reached = [False] * len(blocks)
    reached[0] = True
    work = [0]
    while work:
        i = work.pop()
        out = run(i, entry[i])
        for j in succ(i):
            if not reached[j] or (out and not entry[j]):
                reached[j] = True
                entry[j] = entry[j] or out
                work.append(j)
    bad = []
    for i in range(len(blocks)):
        if reached[i]:
            run(i, entry[i], bad)
    return bad


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_inline_asm_load_returns_into_registers(src):
    bad = {n: b for n, body in _kernels(_asm(src)) if (b := _asm_loads_with_result(body))}
    assert not bad, bad


@pytest.mark.parametrize("src,pattern", [("gemm.hip", "gemm_dl_kernel"),
                                         ("attention.hip", "attn_dkdv_dl_kernel"),
                                         ("attention.hip", "attn_dq_dl_kernel"),
                                         ("attention.hip", "attn_fwd_pp_kernel")])
def test_no_compiler_vmcnt_wait_with_copies_in_flight(src, pattern):
    kernels = _kernels(_asm(src), pattern)
    with_copies = [(n, b) for n, b in kernels if any(c.startswith("global_load_lds") for _, c in _lines(b))]
    assert with_copies, f"no {pattern} kernel with copies found"
    bad = {n: d for n, b in with_copies if (d := _drains_of_copies(b))}
    assert not bad, bad


def test_checkers_catch_planted_cases():
    asm_load = [";;#ASMSTART", "ds_read_b128 v[10:13], v5", ";;#ASMEND"]
    assert _asm_loads_with_result(asm_load)
    asm_tr = [";;#ASMSTART", "ds_read_b64_tr_b16 v[10:11], v5 offset:256", ";;#ASMEND"]
    assert _asm_loads_with_result(asm_tr)
    asm_copy = [";;#ASMSTART", "s_nop 0", "global_load_lds_dwordx4 v[2:3], off", ";;#ASMEND"]
    assert not _asm_loads_with_result(asm_copy)
    compiler_load = ["ds_read_b128 v[10:13], v5", "global_load_dwordx4 v[0:3], v[4:5], off"]
    assert not _asm_loads_with_result(compiler_load)

    copy = [";;#ASMSTART", "global_load_lds_dwordx4 v[2:3], off", ";;#ASMEND"]
    own_wait = [";;#ASMSTART", "s_waitcnt vmcnt(0)", ";;#ASMEND"]
    # a compiler wait between the copies and the loop's own wait drains them
    drained = ["s_mov_b32 s0, 0", ".LBB0_1:"] + own_wait + ["s_barrier"] + copy + [
        "s_waitcnt vmcnt(0)", "ds_read_b128 v[10:13], v5", "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert _drains_of_copies(drained) == ["s_waitcnt vmcnt(0)"]
    # the loop's own waits, and compiler waits once its own vmcnt(0) retired
    # every copy, are fine
    clean = ["s_mov_b32 s0, 0", ".LBB0_1:"] + own_wait + ["s_barrier"] + copy + [
        "ds_read_b128 v[10:13], v5", "s_waitcnt lgkmcnt(0)"] + own_wait + [
        "s_waitcnt vmcnt(0)", "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert not _drains_of_copies(clean)
    # at the loop head the previous trip's copies may still be in flight
    head = ["s_mov_b32 s0, 0", ".LBB0_1:", "s_waitcnt vmcnt(0)"] + own_wait + copy + [
        "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert _drains_of_copies(head) == ["s_waitcnt vmcnt(0)"]
    # after a loop that may exit with copies in flight, a compiler wait in
    # the code that follows drains them; one after an own wait does not
    tail = ["s_mov_b32 s0, 0", ".LBB0_1:"] + own_wait + copy + ["s_cbranch_scc1 .LBB0_1",
                                                                "global_load_dword v1, v[2:3], off",
                                                                "s_waitcnt vmcnt(0)", "s_endpgm"]
    assert _drains_of_copies(tail) == ["s_waitcnt vmcnt(0)"]
    tail_ok = tail[:-3] + own_wait + tail[-3:]
    assert not _drains_of_copies(tail_ok)
    # a branch around the copies still counts the path through them
    skip = ["s_cbranch_scc0 .LBB0_2"] + copy + [".LBB0_2:", "s_waitcnt vmcnt(0)", "s_endpgm"]
    assert _drains_of_copies(skip) == ["s_waitcnt vmcnt(0)"]
    # no copies, no finding
    plain = [".LBB0_1:", "global_load_dword v1, v[2:3], off", "s_waitcnt vmcnt(0)",
             "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert not _drains_of_copies(plain)
