"""Wait states after the hand-issued matrix-core instructions, checked in this
build's own gfx950 assembly (CPU only: hipcc -S, no GPU).

The tile kernels issue v_mfma_* from inline assembly, so the compiler does
not know their latency: every path that leaves a main loop runs a drain of
hand-placed s_nop wait states before any accumulator is read.  A missed
drain gives wrong sums on the GPU, not an error.  This test walks the
control-flow graph of every tile kernel and, for every instruction that reads
or writes an accumulator register (AGPR) that an inline-assembly matrix-core
instruction wrote, takes the fewest wait states (one per instruction, N + 1
per s_nop N) on any path back to that write.  It must be at least 20: an
XDL write of a register and a vector read of it need passes + 3 wait states
on CDNA3 and one more on gfx950, and the longest of these instructions has 16
passes.  Matrix-core instructions that accumulate into the same registers
(source C) are exempt: the hardware chains those.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a8_quantized_gemm_amd", "csrc")
OUT = os.path.join(ROOT, "tests", "sanitize", "_build")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
SOURCES = ("gemm_mfma16.hip", "gemm_mfma.hip", "gemm_fp8_mfma.hip")
REQUIRED = 20
CAP = 1 << 20  # "no pending write"


def _asm(src):
    out = os.path.join(OUT, "hz_" + os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--offload-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return open(out).read()


def _regs(tok, kind):
    """Register numbers of kind 'a' or 'v' named by one operand token."""
    m = re.fullmatch(kind + r"\[(\d+):(\d+)\]", tok)
    if m:
        return list(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(kind + r"(\d+)", tok)
    return [int(m.group(1))] if m else []


def _functions(asm):
    """{name: [(mnemonic, operands, from_inline_asm, label_or_None)]}."""
    funcs = {}
    for body in re.split(r"\n(?=_Z\S+:)", asm):
        name = body.split(":", 1)[0]
        if not name.startswith("_Z"):
            continue
        items, in_asm = [], False
        for line in body.split("\n")[1:]:
            s = line.strip()
            if s.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if s.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if s.startswith(".Lfunc_end"):
                break
            m = re.match(r"^(\.LBB\d+_\d+):", s)
            if m:
                items.append((None, [], False, m.group(1)))
                continue
            if not s or s.startswith((";", ".")) or s.endswith(":"):
                continue
            s = s.split(";")[0].strip()
            parts = s.split(None, 1)
            ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
            items.append((parts[0], ops, in_asm, None))
        funcs[name] = items
    return funcs


def _blocks(items):
    """Basic blocks and their successor indices.  A label maps to the next
    block that has instructions (consecutive labels share it)."""
    blocks, cur, labels = [], [], {}
    for mn, ops, hand, label in items:
        if label is not None:
            if cur:
                blocks.append(cur)
            cur = []
            labels[label] = len(blocks)
            continue
        cur.append((mn, ops, hand))
        if mn.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    succ = []
    for i, b in enumerate(blocks):
        mn, ops, _ = b[-1] if b else ("", [], False)
        s = []
        if mn.startswith(("s_branch", "s_cbranch")):
            s.append(labels[ops[0]])
        if not mn.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def _check(items):
    """Fewest wait states between a hand-issued matrix-core write of an AGPR
    and a later access of it; returns (minimum, list of violations)."""
    blocks, succ = _blocks(items)
    entry = [dict() for _ in blocks]  # AGPR -> wait states since its pending write
    done = [False] * len(blocks)
    seen_min, bad = CAP, []

    def run(i, state, record):
        nonlocal seen_min
        st = dict(state)
        for mn, ops, hand in blocks[i]:
            if mn.startswith("v_mfma") and hand:
                # its source-C read of the same registers is chained
                for tok in ops[1:3]:
                    for a in _regs(tok, "a"):
                        if a in st:
                            if record:
                                seen_min = min(seen_min, st[a])
                                if st[a] < REQUIRED:
                                    bad.append((mn, ops, st[a]))
            else:
                touched = [a for tok in ops for a in _regs(tok, "a")]
                for a in touched:
                    if a in st:
                        if record:
                            seen_min = min(seen_min, st[a])
                            if st[a] < REQUIRED:
                                bad.append((mn, ops, st[a]))
                if not mn.startswith("v_mfma"):
                    for a in _regs(ops[0], "a") if ops else []:
                        st.pop(a, None)  # rewritten by a tracked instruction
            step = int(ops[0]) + 1 if mn == "s_nop" else 1
            for a in list(st):
                st[a] = min(CAP, st[a] + step)
                if st[a] >= 64:
                    del st[a]  # far past any requirement
            if mn.startswith("v_mfma") and hand:
                for a in _regs(ops[0], "a"):
                    st[a] = 0  # wait states are counted from the next instruction
        return st

    work = [0] if blocks else []
    while work:
        i = work.pop()
        done[i] = True
        out = run(i, entry[i], False)
        for j in succ[i]:
            merged = dict(entry[j])
            changed = not done[j]
            for a, d in out.items():
                if d < merged.get(a, CAP):
                    merged[a] = d
                    changed = True
            if changed:
                entry[j] = merged
                work.append(j)
    for i in range(len(blocks)):
        if done[i]:
            run(i, entry[i], True)
    return seen_min, bad


@pytest.fixture(scope="module")
def funcs():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(3) as ex:
        asms = list(ex.map(_asm, SOURCES))
    out = {}
    for a in asms:
        out.update(_functions(a))
    return out


def test_every_tile_kernel_is_checked(funcs):
    hand = [n for n, items in funcs.items()
            if any(mn and mn.startswith("v_mfma") and h for mn, _, h, _ in items)]
    # the 16 x 16 x 64, 32 x 32 x 32 and FP8 tile kernels, every instance
    assert any("w4a8_mfma16_kernel" in n for n in hand)
    assert any("w4a8_mfma_kernel" in n for n in hand)
    assert any("w4fp8_mfma_kernel" in n for n in hand)
    assert len(hand) >= 40, len(hand)


def test_accumulator_reads_follow_the_drain(funcs):
    for name, items in funcs.items():
        if not any(mn and mn.startswith("v_mfma") and h for mn, _, h, _ in items):
            continue
        _, bad = _check(items)
        assert not bad, (name, bad[:4])


def test_checker_finds_a_missing_drain():
    """The check itself: a matrix-core write read back after too few wait
    states is reported, on a straight path and around a loop."""
    def prog(lines):
        return _functions("_Zk:\n" + "\n".join(lines) + "\n.Lfunc_end0:\n")["_Zk"]

    mf = ["\t;;#ASMSTART", "\tv_mfma_i32_16x16x64_i8 a[0:3], v[0:3], v[4:7], a[0:3]",
          "\t;;#ASMEND"]
    ok = mf + ["\ts_nop 7", "\ts_nop 7", "\ts_nop 7", "\ts_nop 7",
               "\tv_accvgpr_read_b32 v8, a2", "\ts_endpgm"]
    short = mf + ["\ts_nop 7", "\ts_nop 7", "\tv_accvgpr_read_b32 v8, a2", "\ts_endpgm"]
    assert _check(prog(ok))[1] == []
    assert len(_check(prog(short))[1]) == 1
    # the write sits at the bottom of a loop whose exit reads at once; the
    # drain is only on the fall-through path of another branch
    loop = [".LBB0_1:"] + mf + ["\ts_cbranch_scc1 .LBB0_1", "\ts_cbranch_vccz .LBB0_2",
                                "\ts_nop 7", "\ts_nop 7", "\ts_nop 7", ".LBB0_2:",
                                "\tv_accvgpr_read_b32 v8, a0", "\ts_endpgm"]
    assert len(_check(prog(loop))[1]) >= 1
    # chained accumulation needs no wait
    chain = mf + mf + ["\ts_nop 7", "\ts_nop 7", "\ts_nop 7", "\ts_nop 7",
                       "\tv_accvgpr_read_b32 v8, a1", "\ts_endpgm"]
    assert _check(prog(chain))[1] == []
