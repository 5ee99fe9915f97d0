"""CPU check of the compiled GEMM kernels: inline-assembly loads are safe.

Some loads in the prefill GEMMs are issued from inline assembly (direct
global->LDS copies, LDS reads into AGPRs), so the compiler does not track them.
Its waits are tied to the loaded values, which keeps every use of a value
behind the wait. This test compiles the kernels to gfx950 assembly with the
library's own flags. It then checks that no instruction writes a register
while a load into that register is still in flight (a late write by the load
would clobber an unrelated value, an address for instance), and that no
instruction reads such a register before the load has landed (it would see a
stale value: an MFMA operand, a copy out of an AGPR, a spill).

The scan is linear over each kernel body; every group of the main loop ends
with a full wait, so no load is in flight across the loop edge.
"""
import os
import re
import shutil
import subprocess

import pytest

from bit_packed_weight_amd import _build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


SOURCE_ONLY = ("global_store", "ds_write", "buffer_store", "global_load_lds", "flat_store", "scratch_store")


def writes_before_wait(body):
    """Instructions that write a register an in-flight load will still write, or
    read a register before the in-flight load into it has landed."""
    vm, lgkm, bad = [], [], []
    for no, line in enumerate(body):
        if not line or line.startswith((";", ".")) or line.endswith(":"):
            continue
        op = line.split()[0]
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", line)
            if m:
                n = int(m.group(1))
                vm = vm[len(vm) - n:] if n else []
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                n = int(m.group(1))
                lgkm = lgkm[len(lgkm) - n:] if n else []
            continue
        ops = _operands(line)
        writes, reads = set(), set()
        if ops and not op.startswith(("s_",) + SOURCE_ONLY):
            writes = _regs(ops[0])
            srcs = ops[1:]
        else:
            srcs = ops
        for tok in srcs:
            reads |= _regs(tok.split()[0]) if tok else set()
        for dst, at, text in vm + lgkm:
            if dst & writes:
                bad.append(f"line {no}: {line}  (writes a register loaded since line {at}: {text})")
            elif dst & reads:
                bad.append(f"line {no}: {line}  (reads a register loaded since line {at}: {text})")
        if op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            loads_reg = op.startswith("global_load") and not op.startswith("global_load_lds")
            vm.append((_regs(ops[0]) if loads_reg else set(), no, line))
        elif op.startswith("ds_"):
            lgkm.append((_regs(ops[0]) if op.startswith("ds_read") else set(), no, line))
    return bad


def compile_asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [_build.hipcc(), *_build.COMMON, *_build.DEVICE, *_build.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out.read_text()


def kernel_bodies(asm, pattern):
    names = [n for n in re.findall(r"^(_Z[^:\s]*):", asm, re.M) if re.search(pattern, n)]
    for name in names:
        start = asm.find(name + ":")
        yield name, [line.strip() for line in asm[start:asm.find(".Lfunc_end", start)].splitlines()]


@pytest.mark.parametrize("src,pattern", [("gemm_i8.hip", "gemm_t2_kernel"), ("gemm_i8.hip", "gemm_g_kernel"),
                                         ("gemm_w4.hip", "gemm_w4_kernel")])
def test_no_register_reuse_under_inflight_loads(src, pattern, tmp_path):
    asm = compile_asm(src, tmp_path)
    found = 0
    for name, body in kernel_bodies(asm, pattern):
        found += 1
        bad = writes_before_wait(body)
        assert not bad, f"{name}:\n" + "\n".join(bad[:10])
    assert found > 0


def test_checker_flags_a_clobbered_destination():
    # a register written while a load into it is in flight, then waited: flagged
    body = ["global_load_ushort v7, v[2:3], off", "v_add_u32_e32 v7, 1, v8", "s_waitcnt vmcnt(0)"]
    assert writes_before_wait(body)
    # the same write after the wait: clean
    body = ["global_load_ushort v7, v[2:3], off", "s_waitcnt vmcnt(0)", "v_add_u32_e32 v7, 1, v8"]
    assert not writes_before_wait(body)
    # an AGPR LDS read overwritten before lgkmcnt: flagged
    body = ["ds_read_b128 a[0:3], v1", "v_accvgpr_write_b32 a2, v5", "s_waitcnt lgkmcnt(0)"]
    assert writes_before_wait(body)
    # its destination read before the wait (an MFMA operand, a copy out of it): flagged
    body = ["ds_read_b128 a[0:3], v1", "v_mfma_i32_32x32x32_i8 v[0:15], a[0:3], v[20:23], 0", "s_waitcnt lgkmcnt(0)"]
    assert writes_before_wait(body)
    body = ["ds_read_b128 a[4:7], v1", "v_accvgpr_read_b32 v9, a6", "s_waitcnt lgkmcnt(0)"]
    assert writes_before_wait(body)
    body = ["global_load_dwordx4 v[8:11], v[2:3], off", "global_store_dword v[4:5], v9, off", "s_waitcnt vmcnt(0)"]
    assert writes_before_wait(body)
    # the same reads after the wait, and reads of other registers before it: clean
    body = ["ds_read_b128 a[0:3], v1", "v_accvgpr_read_b32 v9, a6", "s_waitcnt lgkmcnt(0)",
            "v_mfma_i32_32x32x32_i8 v[0:15], a[0:3], v[20:23], 0"]
    assert not writes_before_wait(body)


def test_no_bit_cast_of_a_vector_component():
    # The ROCm clang used here miscompiles __builtin_bit_cast applied directly
    # to an ext_vector component (v.y, v.z, ... are read as v.x); a component
    # must pass through a named scalar first. The kernel sources must not
    # contain the direct form.
    bad = []
    pat = re.compile(r"__builtin_bit_cast\(\s*[^,()]+,\s*[A-Za-z_][\w\[\]]*\.[xyzw]\s*\)")
    for name in sorted(os.listdir(_build.CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(_build.CSRC, name)) as f:
                for no, line in enumerate(f, 1):
                    if pat.search(line):
                        bad.append(f"{name}:{no}: {line.strip()}")
    assert not bad, "\n".join(bad)
    assert pat.search("x = __builtin_bit_cast(h2, v.y);") and not pat.search("__builtin_bit_cast(h2, v1)")
