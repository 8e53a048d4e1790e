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


def basic_blocks(asm, name):
    """The kernel's basic blocks in layout order: [(label, instructions)] and
    the successor indices of each (branch targets and fall-through)."""
    a = asm.index(name + ":")
    b = asm.index(".Lfunc_end", a)
    blocks = [["<entry>", []]]
    for raw in asm[a:b].split("\n")[1:]:
        m = re.match(r"^\s*(\.LBB\S+):", raw) or re.match(r"^\s*;\s*(%bb\.\d+):", raw)
        if m:
            blocks.append([m.group(1), []])
            continue
        line = raw.split(";")[0].strip()
        if line and not line.startswith("."):
            blocks[-1][1].append(line)
    index = {lab: i for i, (lab, _) in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        out, falls = set(), True
        for l in ins:
            op = l.split()[0]
            if op.startswith("s_cbranch"):
                out.add(index[l.split()[-1]])
            elif op == "s_branch":
                out.add(index[l.split()[-1]])
                falls = False
            elif op in ("s_endpgm", "s_setpc_b64"):
                falls = False
        if falls and i + 1 < len(blocks):
            out.add(i + 1)
        succ.append(out)
    return blocks, succ


def block_loop(blocks, succ):
    """Indices of the blocks on the cycle through the first block that holds
    matrix products (the block loop)."""
    first = next(i for i, (_, ins) in enumerate(blocks) if any(l.startswith("v_mfma") for l in ins))
    def reach(start, edges):
        seen, todo = {start}, [start]
        while todo:
            for j in edges[todo.pop()]:
                if j not in seen:
                    seen.add(j)
                    todo.append(j)
        return seen
    pred = [set() for _ in blocks]
    for i, out in enumerate(succ):
        for j in out:
            pred[j].add(i)
    return reach(first, succ) & reach(first, pred)


def d128_kernels(asm):
    for name in re.findall(r"^(_ZN\S*fa_bwd_dkdvILi128E\S*):", asm, re.M):
        blocks, succ = basic_blocks(asm, name)
        yield name, blocks, succ, block_loop(blocks, succ)


def test_dkdv_d128_products_keep_their_registers(device_asm):
    found = 0
    for name, blocks, succ, loop in d128_kernels(device_asm):
        found += 1
        body = [l for i in loop for l in blocks[i][1]]
        mf = [l for l in body if l.startswith("v_mfma")]
        assert len(mf) == 64, (name, len(mf))   # one block: 4 phases x 8 steps x 2
        moves = [l for l in body if l.startswith("v_accvgpr")]
        assert not moves, (name, "register-file copies inside the block loop", moves[:4])
    assert found == 5   # causal x varlen, and the dense non-causal instance with no mask
    for name, lines in kernels(device_asm, "fa_bwd_dkdvILi128E"):
        # the epilogue reads the AGPR accumulators only after the result wait
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        first_read = next(i for i, l in enumerate(lines) if i > mf[-1] and
                          l.startswith("v_accvgpr_read"))
        nops = [l for l in lines[mf[-1]:first_read] if l.startswith("s_nop 15")]
        assert len(nops) >= 2, (name, "no result wait before the accumulators are read")


def test_dkdv_first_products_wait_before_softmax_reads(device_asm):
    """Each phase whose VALU work reads S/dP starts with the 32-state wait."""
    for name, blocks, succ, loop in d128_kernels(device_asm):
        waits = 0
        for i in loop:
            ins = blocks[i][1]
            waits += sum(1 for a, b in zip(ins, ins[1:]) if a == "s_nop 15" and b == "s_nop 15")
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


def _walk(blocks, edges, bi, pos, forward, visit, limit):
    """Visit instructions from block bi, position pos (exclusive), along every
    control-flow path, forwards or backwards, with the wait states passed so
    far; visit(line, ws) returns True to stop that path."""
    todo = [(bi, pos, 0)]
    seen = set()
    while todo:
        b, p, ws = todo.pop()
        ins = blocks[b][1]
        rng = range(p + 1, len(ins)) if forward else range(p - 1, -1, -1)
        stopped = False
        for k in rng:
            if visit(ins[k], ws) or ws >= limit:
                stopped = True
                break
            ws += _wait_states(ins[k])
        if stopped:
            continue
        for nb in edges[b]:
            key = (nb, ws)
            if key not in seen:
                seen.add(key)
                todo.append((nb, -1 if forward else len(blocks[nb][1]), ws))


def test_dkdv_d128_operand_and_result_distances(device_asm):
    """No hazard hides between the inline-assembly products and the VALU code,
    on any control-flow path: a VGPR written by a VALU instruction is read as
    an operand of an AGPR-accumulator product no sooner than 8 wait states
    later (one step of the block body apart, by construction), and a VGPR
    result of a product is touched by non-matrix code no sooner than 32 wait
    states later (the waits that bind S and dP)."""
    for name, blocks, succ, loop in d128_kernels(device_asm):
        pred = [set() for _ in blocks]
        for i, out in enumerate(succ):
            for j in out:
                pred[j].add(i)
        for bi, (_, ins) in enumerate(blocks):
            for k, line in enumerate(ins):
                if not line.startswith("v_mfma"):
                    continue
                ops = _operands(line)
                if ops[0].startswith("a["):
                    srcs = _regs(ops[1]) | _regs(ops[2])

                    def before(t, ws, srcs=srcs, line=line):
                        op = t.split()[0]
                        if op.startswith("v_") and not op.startswith("v_mfma") and \
                                _regs(_operands(t)[0]) & srcs:
                            assert ws >= 8, (name, "VALU write too close to product", t, line)
                            return True
                        return False
                    _walk(blocks, pred, bi, k, False, before, 400)
                elif ops[0].startswith("v["):
                    dst = _regs(ops[0])

                    def after(t, ws, dst=dst, line=line):
                        op = t.split()[0]
                        if not op.startswith("v_mfma") and op.startswith(("v_", "ds_", "global_")):
                            used = set()
                            for x in _operands(t):
                                used |= _regs(x)
                            if used & dst:
                                assert ws >= 32, (name, "product result read too soon", line, t)
                                return True
                        return False
                    _walk(blocks, succ, bi, k, True, after, 32)


def test_dkdv_entry_mask_takes_no_exec_mask_branch(device_asm):
    """The per-entry causal/length mask is a compare and a select, skipped on
    blocks that need none by a wave-uniform (scalar) branch: no exec-mask
    branch shares a block with the products, the exponentials or the
    selects (a two-sided test written with && was once compiled into one
    such branch per entry, a third of the body's instructions)."""
    for name, blocks, succ, loop in d128_kernels(device_asm):
        for i in loop:
            ops = [l.split()[0] for l in blocks[i][1]]
            divergent = any(op.startswith("s_and_saveexec") or op.startswith("s_cbranch_exec")
                            for op in ops)
            stream = any(op.startswith(("v_mfma", "v_exp_f32", "v_cndmask")) for op in ops)
            assert not (divergent and stream), (name, blocks[i][0])
