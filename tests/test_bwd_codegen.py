"""The dK/dV kernel's explicit-register products stay safe (CPU only).

For D = 128 the backward's dK/dV kernel issues its matrix products as
inline assembly with the accumulators pinned to AGPRs (more than 256
registers per lane are live).  The compiler's hazard tracking does not see
inside those statements, so they are only correct while the compiler never
moves their accumulators between register files inside the block loop, and
while the products' results are waited for before anything reads them.
This test compiles the kernels for gfx950 and checks both on the generated
code, so a compiler or source change that breaks them fails here rather
than as wrong gradients on the GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_forward_04_amd import build as fa_build

HIPCC = fa_build.HIPCC


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "fa_bwd.s")
    cmd = [HIPCC, "--offload-arch=" + fa_build.ARCH, "-O3", "-std=c++17", "--cuda-device-only",
           "-S", "-I" + os.path.join(fa_build.ROOT, "include"), "-I" + fa_build.CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-inline-asm",
           "-o", out, os.path.join(fa_build.CSRC, "fa_bwd.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return open(out).read()


def kernels(asm, pattern):
    for name in re.findall(r"^(_ZN\S*" + pattern + r"\S*):", asm, re.M):
        a = asm.index(name + ":")
        b = asm.index(".Lfunc_end", a)
        lines = [l.split(";")[0].strip() for l in asm[a:b].split("\n")]
        yield name, [l for l in lines if l and not l.startswith(".")]


def test_dkdv_d128_products_keep_their_registers(device_asm):
    found = 0
    for name, lines in kernels(device_asm, "fa_bwd_dkdvILi128E"):
        found += 1
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        assert len(mf) == 64, (name, len(mf))   # one block: 4 phases x 8 steps x 2
        inside = [l for l in lines[mf[0]:mf[-1] + 1] if l.startswith("v_accvgpr")]
        assert not inside, (name, "register-file copies inside the block loop", inside[:4])
        # the epilogue reads the AGPR accumulators only after the result wait
        first_read = next(i for i, l in enumerate(lines) if i > mf[-1] and
                          l.startswith("v_accvgpr_read"))
        nops = [l for l in lines[mf[-1]:first_read] if l.startswith("s_nop 15")]
        assert len(nops) >= 2, (name, "no result wait before the accumulators are read")
    assert found == 5   # causal x varlen, and the dense non-causal instance with no mask


def test_dkdv_first_products_wait_before_softmax_reads(device_asm):
    """Each phase whose VALU work reads S/dP starts with the 32-state wait."""
    for name, lines in kernels(device_asm, "fa_bwd_dkdvILi128E"):
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        body = lines[mf[0]:mf[-1] + 1]
        waits = sum(1 for a, b in zip(body, body[1:]) if a == "s_nop 15" and b == "s_nop 15")
        assert waits >= 2, (name, waits)


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(line):
    op = line.split()[0]
    return int(line.split()[1]) + 1 if op == "s_nop" else 1


def test_dkdv_d128_operand_and_result_distances(device_asm):
    """No hazard hides between the inline-assembly products and the VALU code:
    a VGPR written by a VALU instruction is read as an operand of an
    AGPR-accumulator product no sooner than 8 wait states later (one step
    of the block body apart, by construction), and a VGPR result of a
    product is touched by non-matrix code no sooner than 32 wait states
    later (the waits that bind S and dP)."""
    for name, lines in kernels(device_asm, "fa_bwd_dkdvILi128E"):
        lines = [l for l in lines if not l.endswith(":")]
        for i, line in enumerate(lines):
            if not line.startswith("v_mfma"):
                continue
            ops = _operands(line)
            if ops[0].startswith("a["):
                srcs = _regs(ops[1]) | _regs(ops[2])
                ws = 0
                for j in range(i - 1, max(0, i - 400), -1):
                    t = lines[j]
                    op = t.split()[0]
                    if op.startswith("v_") and not op.startswith("v_mfma") and \
                            _regs(_operands(t)[0]) & srcs:
                        assert ws >= 8, (name, "VALU write too close to product", t, line)
                        break
                    ws += _wait_states(t)
            elif ops[0].startswith("v["):
                dst = _regs(ops[0])
                ws = 0
                for t in lines[i + 1:i + 600]:
                    op = t.split()[0]
                    if op.startswith(("s_cbranch", "s_branch")):
                        break
                    if not op.startswith("v_mfma") and op.startswith(("v_", "ds_", "global_")):
                        used = set()
                        for x in _operands(t):
                            used |= _regs(x)
                        if used & dst:
                            assert ws >= 32, (name, "product result read too soon", line, t)
                            break
                    ws += _wait_states(t)


def test_dkdv_entry_mask_is_branch_free(device_asm):
    """The per-entry causal/length mask of P is a compare and a select: no
    exec-mask branch inside the block body (a two-sided test written with
    && was once compiled into one such branch per entry, a third of the
    body's instructions)."""
    for name, lines in kernels(device_asm, "fa_bwd_dkdvILi128E"):
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        body = [l.split()[0] for l in lines[mf[0]:mf[-1] + 1]]
        assert "s_and_saveexec_b64" not in body, name
        assert not any(op.startswith("s_cbranch") for op in body), name
