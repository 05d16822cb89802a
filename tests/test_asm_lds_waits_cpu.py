"""The tiled and quantised kernels read LDS with inline-asm ds_read instructions
and wait for them with explicit s_waitcnt lgkmcnt statements that take the
destinations as in/out operands. The compiler sees such a destination as
written when the asm statement ends, while the hardware writes it when the
read returns: a copy, spill or reuse of that register before the wait would
read garbage or be overwritten by the late return. This test compiles those
kernels for gfx950 and checks the emitted ISA: on every control-flow path from
an inline-asm LDS read to the first s_waitcnt lgkmcnt(n) that guarantees its
completion (n no larger than the LDS/scalar-memory operations issued after it;
they complete in order), no instruction reads or writes its destination
registers."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from sparse_moe_layer_gemm_amd import build as pkg_build  # noqa: E402

ASM_LDS_FILES = ["expert_tile.hip", "expert_tile_q.hip", "expert_stream_q.hip"]
LGKM_OPS = re.compile(r"^(ds_|s_load|s_buffer_load|s_sendmsg|s_memtime|s_memrealtime|s_get_barrier)")


def _regs(tok):
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def _parse(line):
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    if not parts:
        return "", []
    ops = re.findall(r"[va]\[\d+:\d+\]|[va]\d+", parts[1]) if len(parts) > 1 else []
    return parts[0], ops


def unsafe_asm_lds_reads(text):
    """(asm LDS reads, list of violations) for one ISA listing."""
    ins, labels, in_asm_flags = [], {}, []
    in_asm = False
    for raw in text.split("\n"):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if re.match(r"^\.LBB\d+_\d+:", s) or re.match(r"^_Z\S*:", s):
            labels[s.split(":")[0]] = len(ins)
            ins.append(None)
            in_asm_flags.append(False)
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        ins.append(s)
        in_asm_flags.append(in_asm)
    n, bad = 0, []
    for i, s in enumerate(ins):
        if s is None or not in_asm_flags[i]:
            continue
        op, ops = _parse(s)
        if not op.startswith("ds_read"):
            continue
        n += 1
        dest = _regs(ops[0])
        seen, stack = set(), [(i + 1, 0)]
        while stack:
            j, cnt = stack.pop()
            while j < len(ins):
                if (j, cnt) in seen:
                    break
                seen.add((j, cnt))
                t = ins[j]
                if t is None:
                    j += 1
                    continue
                top, tops = _parse(t)
                if top == "s_waitcnt":
                    m = re.search(r"lgkmcnt\((\d+)\)", t)
                    if m and int(m.group(1)) <= cnt:
                        break
                    j += 1
                    continue
                used = set()
                for o in tops:
                    used |= _regs(o)
                if used & dest:
                    bad.append(f"{s} -> {t}")
                    stack = []
                    break
                if LGKM_OPS.match(top):
                    cnt = min(cnt + 1, 64)
                if top in ("s_endpgm", "s_setpc_b64"):
                    break
                if top.startswith("s_cbranch"):
                    stack.append((labels[t.split()[1]], cnt))
                    j += 1
                    continue
                if top == "s_branch":
                    j = labels[t.split()[1]]
                    continue
                j += 1
    return n, bad


def test_checker_finds_a_planted_early_use():
    listing = """_Zk:
\t;;#ASMSTART
\tds_read_b128 v[10:13], v2
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_2
\tv_add_f32 v5, v6, v7
.LBB0_2:
\tv_mov_b32 v20, {src}
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\ts_endpgm
"""
    assert unsafe_asm_lds_reads(listing.format(src="v11"))[1]  # reads a pending destination
    assert not unsafe_asm_lds_reads(listing.format(src="v14"))[1]


@pytest.mark.parametrize("src", ASM_LDS_FILES)
def test_inline_asm_lds_reads_complete_before_use(src, tmp_path):
    flags = [f for f in pkg_build.FLAGS if f != "-fPIC"]
    out = tmp_path / (src + ".s")
    r = subprocess.run([pkg_build.HIPCC, *flags, "--cuda-device-only", "-S",
                        os.path.join(pkg_build.CSRC, src), "-o", str(out)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    n, bad = unsafe_asm_lds_reads(out.read_text())
    assert n > 0
    assert not bad, bad[:5]
