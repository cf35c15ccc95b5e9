"""The direct global -> LDS tile copies are inline assembly, which the
compiler's hazard checks and its memory-counter bookkeeping do not see.

* A vector instruction that writes an SGPR needs 5 wait states before a
  vector memory instruction reads that SGPR as an address (gfx9), so every
  copy must carry its own s_nop 4.
* The prefill kernels issue the copies of key tiles 0 and 1 and then wait
  with vmcnt(N), N being the copies one tile issues per wave, so that tile
  0's copies have landed while tile 1's may still be in flight.  That wait is
  right only if every way through the code issues exactly N copy
  instructions per tile and no other vector memory instruction after them.

This compiles the library's device code to assembly (no GPU needed) and
checks both in every kernel."""
import os
import re
import subprocess

import pytest

from scaled_dot_product_qk_amd import build as b


@pytest.fixture(scope="module")
def asm_lines(tmp_path_factory):
    return _device_asm(tmp_path_factory.mktemp("asm"))


def _device_asm(tmp_path):
    out = tmp_path / "attn.s"
    cmd = [b.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", b.INCLUDE, "-I", b.CSRC,
           os.path.join(b.CSRC, "attn_api.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: " + res.stderr[-400:])
    return out.read_text().splitlines()


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_every_lds_copy_is_guarded(asm_lines):
    lines = asm_lines
    hist, copies, unguarded, hazards = [], 0, [], []
    for raw in lines:
        line = raw.strip()
        if re.match(r"^_ZN[^:\s]+:", line):
            hist = []
            continue
        if not line or line.startswith((";", ".")) or line.endswith(":"):
            continue
        if line.startswith("global_load_lds"):
            copies += 1
            if not (hist and hist[-1].startswith("s_nop 4")):
                unguarded.append(line)
            base = _sgprs(line.split(None, 1)[1].split(",")[1].strip())
            waits = 0
            for prev in reversed(hist[-12:]):
                op = prev.split()[0]
                if op == "s_nop":
                    waits += int(prev.split()[1]) + 1
                    continue
                if waits >= 5:
                    break
                dst = prev.split(None, 1)[1].split(",")[0].strip() if " " in prev else ""
                if op.startswith("v_") and _sgprs(dst) & base:
                    hazards.append((prev, line, waits))
                waits += 1
        hist.append(line)
    assert copies > 0
    assert not unguarded, unguarded[:3]
    assert not hazards, hazards[:3]


# ---------------------------------------------------------------------------
# The prologue wait of the prefill kernels.

_VMEM = ("global_", "buffer_", "flat_", "scratch_")
MARK = ";;#copy-group-end"  # emitted by copy_group_end() after each group of copies


def _kernels(lines):
    """{kernel symbol: its instruction and label lines}."""
    out, name = {}, None
    for raw in lines:
        line = MARK if MARK in raw else raw.split(";")[0].strip()
        m = re.match(r"^(_ZN[^:\s]+):$", line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name is None or not line:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        if line.startswith(".") and not re.match(r"^\.LBB\d+_\d+:$", line):
            continue
        out[name].append(line)
    return out


def _blocks(body):
    """Basic blocks [(label, [instructions], [successor labels])]."""
    blocks, cur, label = [], [], "entry"
    for line in body:
        if line.endswith(":"):
            blocks.append([label, cur, None])
            label, cur = line[:-1], []
            continue
        cur.append(line)
        op = line.split()[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op in ("s_endpgm", "s_setpc_b64"):
            blocks.append([label, cur, None])
            label, cur = f"{label}+", []
    blocks.append([label, cur, None])
    blocks = [b for b in blocks if b[1] or b[0] != "entry" or True]
    for i, b in enumerate(blocks):
        succ = []
        last = b[1][-1].split() if b[1] else []
        op = last[0] if last else ""
        if op == "s_branch":
            succ = [last[1]]
        elif op.startswith("s_cbranch"):
            succ = [last[1]] + ([blocks[i + 1][0]] if i + 1 < len(blocks) else [])
        elif op not in ("s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            succ = [blocks[i + 1][0]]
        b[2] = succ
    return blocks


def _vmcnt(line):
    m = re.match(r"s_waitcnt\s.*vmcnt\((\d+)\)", line)
    return int(m.group(1)) if m else None


def _regs(tok):
    tok = tok.strip()
    if tok.startswith("vcc"):
        return {"vcc"}
    return {("s", r) for r in _sgprs(tok)}


def _step_consts(consts, line):
    """Track the scalar flags the compiler's structured branches test: a
    register pair set to -1 or 0 by s_mov_b64 and turned into vcc by
    s_andn2_b64/s_and_b64 vcc, exec, <pair>.  exec is never empty here (every
    lane of a wave takes part in the copies), so vcc = exec & ~(-1) is 0 and
    vcc = exec & ~0 is not."""
    if line == MARK:
        return consts
    parts = line.replace(",", " ").split()
    op, args = parts[0], parts[1:]
    c = dict(consts)
    if op == "s_mov_b64" and len(args) == 2 and args[1] in ("-1", "0"):
        for r in _regs(args[0]):
            c.pop(r, None)
        c[args[0]] = int(args[1])
        return c
    if op in ("s_andn2_b64", "s_and_b64") and args[:2] == ["vcc", "exec"] and args[2] in c:
        src = c[args[2]]
        c["vcc"] = (src == 0) if op == "s_andn2_b64" else (src != 0)  # True: vcc nonzero
        return c
    if args and (op.startswith("s_") or op.startswith("v_")) and not op.startswith(("s_cbranch", "s_branch")):
        written = _regs(args[0])
        if op.startswith("v_cmp"):
            written |= {"vcc"}
        for k in list(c):
            if k == "vcc":
                if "vcc" in written:
                    c.pop(k)
            elif _regs(k) & written:
                c.pop(k)
    return c


def _prologue_paths(body):
    """(N, states): N is the immediate of the first nonzero vmcnt wait after
    the kernel's first copy, states the set of (copies since the last group
    marker, sizes of the completed copy groups) over every feasible path
    from the kernel's entry to that wait.  Paths are pruned only where a
    branch tests a flag that the structured control flow set to a constant
    on that path."""
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks)}
    seen_copy, wpos = False, None
    for i, b in enumerate(blocks):
        for j, line in enumerate(b[1]):
            if line.startswith("global_load_lds"):
                seen_copy = True
            n = _vmcnt(line)
            if seen_copy and n and wpos is None:
                wpos = (i, j, n)
    assert wpos is not None, "no prologue wait found"
    wb, wj, N = wpos
    preds = {i: [] for i in range(len(blocks))}
    for i, b in enumerate(blocks):
        for s_ in b[2]:
            if s_ in index:
                preds[index[s_]].append(i)
    reach, todo = {wb}, [wb]
    while todo:
        for p in preds[todo.pop()]:
            if p not in reach:
                reach.add(p)
                todo.append(p)
    assert 0 in reach
    order, visiting, done = [], set(), set()

    def topo(i):  # the blocks before the wait form a DAG
        if i in done:
            return
        assert i not in visiting, "loop before the prologue wait"
        visiting.add(i)
        if i != wb:
            for s_ in blocks[i][2]:
                k = index.get(s_)
                if k is not None and k in reach:
                    topo(k)
        visiting.discard(i)
        done.add(i)
        order.append(i)

    topo(0)
    states = {0: {(0, (), frozenset())}}
    at_wait = set()
    for i in reversed(order):
        lines = blocks[i][1][:wj] if i == wb else blocks[i][1]
        for since, groups, fz in states.get(i, set()):
            consts = dict(fz)
            for line in lines:
                if line == MARK:
                    groups, since = groups + (since,), 0
                    continue
                if line.startswith("global_load_lds"):
                    since += 1
                consts = _step_consts(consts, line)
            if i == wb:
                at_wait.add((since, groups))
                continue
            succ = list(blocks[i][2])
            last = lines[-1].split() if lines else []
            if last and last[0] in ("s_cbranch_vccnz", "s_cbranch_vccz") and "vcc" in consts:
                taken = consts["vcc"] if last[0] == "s_cbranch_vccnz" else not consts["vcc"]
                succ = succ[:1] if taken else succ[1:]
            key = frozenset(consts.items())
            for s_ in succ:
                k = index.get(s_)
                if k is not None and k in reach:
                    states.setdefault(k, set()).add((since, groups, key))
    return N, at_wait


def test_prefill_prologue_wait_counts_one_tile_of_copies(asm_lines):
    """The prologue issues tile 0's copies, then tile 1's, then waits with
    vmcnt(N).  That releases exactly tile 0 if every group of copies holds N
    copy instructions on every way through the code and the wait follows a
    group's end with no copy in between.  (Other vector memory instructions
    among the copies, such as spill reloads, only make the wait stricter.)"""
    kernels = {k: v for k, v in _kernels(asm_lines).items()
               if "attn_fwd_bf16_kernel" in k or "attn_fwd_fp8_kernel" in k}
    assert len(kernels) >= 22
    for name, body in kernels.items():
        assert sum(line == MARK for line in body) >= 3, name
        N, states = _prologue_paths(body)
        assert states, name
        for since, groups in states:
            assert since == 0 and groups, (name, N, since, groups)
            assert all(g == N for g in groups), (name, N, groups)


def test_prologue_check_catches_a_short_group(asm_lines):
    """The check itself: one copy dropped from a kernel's first group, or a
    marker lost so that the wait follows copies of an unfinished group, is
    reported."""
    name, body = next((k, v) for k, v in _kernels(asm_lines).items() if "attn_fwd_bf16_kernel" in k)
    first = next(i for i, line in enumerate(body) if line.startswith("global_load_lds"))
    N, states = _prologue_paths(body[:first] + body[first + 1:])
    assert any(g != N for _, groups in states for g in groups)
    marks = [i for i, line in enumerate(body) if line == MARK]
    N, states = _prologue_paths(body[:marks[1]] + body[marks[1] + 1:])
    assert any(since != 0 or any(g != N for g in groups) for since, groups in states)
