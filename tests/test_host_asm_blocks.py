"""Static checks of the hand-written LDS-read / MFMA asm blocks (CPU only).

The decode ring and the prefill issue their LDS operand reads, and the
prefill its MFMAs, from inline asm that the compiler does not look into, so
the waits, the buffer rotation and the operand wiring are checked here by
reading the source: each block's instruction strings and its operand lists
are parsed and run through a small model of the LDS return queue.

Model: ds_read_b128 / ds_read_b64 go into a FIFO (LDS reads return in
order); `s_waitcnt lgkmcnt(N)` retires the oldest until at most N remain.
An MFMA may only read a buffer whose read has retired; a buffer is not
reloaded while its read is in flight or before an MFMA has used it; every
read retires inside its block.  On top of that each block's data flow is
compared with what the code around it expects the block to compute.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_271_amd", "csrc")


def _source(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


def _split_top(s, sep):
    """Split s at `sep` characters outside parentheses, brackets and strings."""
    out, depth, cur, in_str = [], 0, [], False
    for ch in s:
        if in_str:
            cur.append(ch)
            if ch == '"':
                in_str = False
            continue
        if ch == '"':
            in_str = True
        elif ch in "([":
            depth += 1
        elif ch in ")]":
            depth -= 1
        elif ch == sep and depth == 0:
            out.append("".join(cur))
            cur = []
            continue
        cur.append(ch)
    out.append("".join(cur))
    return out


def asm_block(file, function):
    """(instructions, operands) of the asm volatile block in `function`;
    operands[i] = (constraint, C++ expression) of %i."""
    src = _source(file)
    macros = dict(re.findall(r'#define\s+(\w+)\s+((?:"[^"\n]*"\s*)+)', src))
    start = src.index(function)
    i = src.index("asm volatile(", start) + len("asm volatile(")
    depth, j = 1, i
    while depth:
        depth += {"(": 1, ")": -1}.get(src[j], 0)
        j += 1
    body = src[i:j - 1]
    parts = _split_top(body, ":")
    text = parts[0]
    for name, value in macros.items():
        text = re.sub(r"\b%s\b" % name, value, text)
    code = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', text)).replace("\\n", "\n")
    instrs = [l.strip() for l in code.split("\n") if l.strip()]
    operands = []
    for part in parts[1:3]:
        for item in _split_top(part, ","):
            m = re.match(r'\s*"([^"]*)"\s*\((.*)\)\s*$', item, re.S)
            if m:
                operands.append((m.group(1), re.sub(r"\s+", "", m.group(2))))
    return instrs, operands


def run_model(instrs, operands):
    """Run the block through the LDS-queue model.  Returns (loads, mfmas):
    loads[k] = (dst expression, address expression, byte offset) in issue
    order; mfmas = list of (dst, a, b, c) where a buffer operand is replaced
    by the (address, offset) of the read it holds."""
    name = lambda tok: operands[int(tok[1:])][1] if tok.startswith("%") else tok
    pending = []          # FIFO of dst operand indexes
    holds = {}            # dst operand -> (address, offset) of its retired read
    used = {}             # dst operand -> consumed by an MFMA since its read
    loads, mfmas = [], []
    for ins in instrs:
        op, _, rest = ins.partition(" ")
        args = [a.strip() for a in rest.split(",")] if rest else []
        if op.startswith("ds_read_b"):
            dst = int(args[0][1:])
            addr, _, off = args[1].partition(" offset:")
            assert operands[dst][0] == "=&v", f"{ins}: a read destination must be an early-clobber output"
            assert dst not in pending, f"{ins}: reloads a buffer whose read is in flight"
            if any(o.startswith("v_mfma") for o in (i.split(" ")[0] for i in instrs)):
                assert used.get(dst, True), f"{ins}: reloads a buffer no MFMA has used"
            pending.append(dst)
            holds.pop(dst, None)
            used[dst] = False
            loads.append((operands[dst][1], name(addr), int(off or 0)))
        elif op == "s_waitcnt":
            n = int(re.fullmatch(r"lgkmcnt\((\d+)\)", args[0]).group(1))
            while len(pending) > n:
                retired = pending.pop(0)
                # the retired read is the latest one issued into that buffer
                last = max(k for k, l in enumerate(loads) if l[0] == operands[retired][1])
                holds[retired] = loads[last][1:]
        elif op.startswith("v_mfma"):
            srcs = []
            for tok in args[1:3]:
                if tok.startswith("%") and operands[int(tok[1:])][0] == "=&v":
                    k = int(tok[1:])
                    assert k not in pending, f"{ins}: reads a buffer whose LDS read has not retired"
                    assert k in holds, f"{ins}: reads a buffer that holds no read"
                    used[k] = True
                    srcs.append(holds[k])
                else:
                    srcs.append(name(tok))
            mfmas.append((name(args[0]), srcs[0], srcs[1], name(args[3])))
        elif op == "s_nop":
            pass
        else:
            raise AssertionError(f"unexpected instruction {ins!r}")
    assert not pending, "reads still in flight at the end of the block"
    return loads, mfmas


def wait_states(instrs):
    """Wait states of the leading and of the trailing s_nop run."""
    def run(seq):
        n = 0
        for ins in seq:
            m = re.fullmatch(r"s_nop (\d+)", ins)
            if not m:
                break
            n += int(m.group(1)) + 1
        return n
    return run(instrs), run(instrs[::-1])


def check_scores(instrs, ops):
    loads, mfmas = run_model(instrs, ops)
    # read 2 kk + j: K operand of k-step kk, keys 4 j .., from a_kk + 1024 j
    assert sorted((a, off) for _, a, off in loads) == sorted((f"a{kk}", 1024 * j) for kk in range(4) for j in range(2))
    seen = {}
    for d, a, b, c in mfmas:
        m = re.fullmatch(r"S\[(\d)\]\[0\]\[(\d)\]", d)
        assert m, d
        rt, j = int(m.group(1)), int(m.group(2))
        (addr, off) = a
        kk = int(addr[1:])
        assert off == 1024 * j, f"S[{rt}][0][{j}] takes keys of the other half: {a}"
        assert b == f"t.qv[{rt}][{kk}]", f"S[{rt}][0][{j}] k-step {kk} multiplies {b}"
        first = (rt, j) not in seen
        assert c == ("0" if first else d), f"S[{rt}][0][{j}] accumulator {c}"
        seen.setdefault((rt, j), []).append(kk)
    assert {k: sorted(v) for k, v in seen.items()} == {(rt, j): [0, 1, 2, 3] for rt in range(2) for j in range(2)}
    lead, tail = wait_states(instrs)
    assert lead >= 2 and tail >= 18


def test_prefill_scores_block():
    check_scores(*asm_block("prefill.hip", "void chunk_scores128("))


def check_pv(instrs, ops):
    loads, mfmas = run_model(instrs, ops)
    # read t8: V operand of output dims 16 t8 .., from av + 512 t8
    assert sorted((a, off) for _, a, off in loads) == [("av", 512 * t8) for t8 in range(8)]
    seen = set()
    for d, a, b, c in mfmas:
        m = re.fullmatch(r"t\.acc\[(\d)\]\[(\d)\]", d)
        assert m, d
        rt, t8 = int(m.group(1)), int(m.group(2))
        assert a == ("av", 512 * t8), f"acc[{rt}][{t8}] takes V tile {a}"
        assert b == f"pop[{rt}][0]" and c == d
        assert (rt, t8) not in seen
        seen.add((rt, t8))
        assert ops[[o[1] for o in ops].index(d)][0] == "+v"
    assert seen == {(rt, t8) for rt in range(2) for t8 in range(8)}
    lead, tail = wait_states(instrs)
    assert lead >= 2 and tail >= 18


def test_prefill_pv_block():
    check_pv(*asm_block("prefill.hip", "void chunk_pv128("))


@pytest.mark.parametrize("function,expect", [
    # bf16 ring: K operand [j][kk] at a_kk + 1024 j, V slice i at av + 512 i
    ("void ring_read(", {**{f"kop[{j}][{kk}]": (f"a{kk}", 1024 * j) for j in range(2) for kk in range(4)},
                         **{f"vr[{i}]": ("av", 512 * i) for i in range(8)}}),
    # 8-bit ring: K granules [j][s] at a_{2j+s}, V half rows i at av + 256 i, the scales at as
    ("void ring_read8(", {**{f"kseg[{j}][{s}]": (f"a{2 * j + s}", 0) for j in range(2) for s in range(2)},
                          **{f"vr[{i}]": ("av", 256 * i) for i in range(8)}, "sc": ("as", 0)}),
])
def test_decode_ring_read_blocks(function, expect):
    instrs, ops = asm_block("decode.hip", function)
    loads, mfmas = run_model(instrs, ops)
    assert not mfmas
    assert {d: (a, off) for d, a, off in loads} == expect
    assert len(loads) == len(expect), "an output is read twice"


def test_model_catches_planted_mistakes():
    """The checks fail a wait one short, a block that ends with a read in
    flight, a wrong q k-step, a V tile fed to the wrong output and a short
    tail of wait states."""
    def planted(instrs, old, new):
        assert old in instrs, old
        k = instrs.index(old)
        return instrs[:k] + [new] + instrs[k + 1:]
    pv, pv_ops = asm_block("prefill.hip", "void chunk_pv128(")
    with pytest.raises(AssertionError, match="not retired"):
        check_pv(planted(pv, "s_waitcnt lgkmcnt(2)", "s_waitcnt lgkmcnt(3)"), pv_ops)
    with pytest.raises(AssertionError):
        check_pv(planted(pv, "s_waitcnt lgkmcnt(0)", "s_waitcnt lgkmcnt(1)"), pv_ops)
    with pytest.raises(AssertionError, match="takes V tile"):
        check_pv(planted(pv, "v_mfma_f32_16x16x32_bf16 %3, %16, %19, %3", "v_mfma_f32_16x16x32_bf16 %2, %16, %19, %2"),
                 pv_ops)
    with pytest.raises(AssertionError):
        check_pv([i for i in pv if i != "s_nop 1"], pv_ops)
    sc, sc_ops = asm_block("prefill.hip", "void chunk_scores128(")
    with pytest.raises(AssertionError, match="multiplies"):
        check_scores(planted(sc, "v_mfma_f32_16x16x32_bf16 %1, %4, %8, %1", "v_mfma_f32_16x16x32_bf16 %1, %4, %9, %1"),
                     sc_ops)
    with pytest.raises(AssertionError, match="accumulator"):
        check_scores(planted(sc, "v_mfma_f32_16x16x32_bf16 %0, %6, %8, %0", "v_mfma_f32_16x16x32_bf16 %0, %6, %8, 0"),
                     sc_ops)
