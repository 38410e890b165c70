"""The hand-written MFMAs of the d >= 192 dK/dV kernels (CPU: reads gfx950 assembly).

Those kernels keep their dK/dV accumulators in AGPRs through MFMAs written as
inline asm, which the compiler's hazard recognizer does not see: the wait states
it would place are written into the asm itself (two before each group of MFMAs,
a settle of 16 after each step's last group).  That is only sufficient if the
code the compiler emits around them has a certain shape, and nothing in the
source can force it, so this test compiles the unit exactly as the build does
and checks it:

* every run of hand-written MFMAs is straight-line code (no label or branch) that
  ends in the settle;
* no compiler-placed instruction reads or writes the accumulator AGPRs inside
  such a run.

Everything else that touches those AGPRs (the zero fills of a new item, the
copies the compiler places where loop paths join, the epilogue) then follows a
settle on every path.  Planted violations (on text, not on a GPU) check that the
checker sees them.
"""
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from bwd_varlen_flashattention_amd import build  # noqa: E402

KERNEL = re.compile(r"^(_ZN3jfa15bwd_dkdv_kernel\S+):\s.*?\n(.*?)s_endpgm", re.S | re.M)
SETTLE = "s_nop 15"


def _agprs(text):
    regs = set()
    for lo, hi in re.findall(r"\ba\[(\d+):(\d+)\]", text):
        regs.update(range(int(lo), int(hi) + 1))
    regs.update(int(x) for x in re.findall(r"\ba(\d+)\b", text))
    return regs


def check_kernel(body):
    """Returns (number of hand-written MFMAs, number of settles, list of violations)."""
    lines = body.splitlines()
    in_asm, asm_line, acc = False, set(), set()
    for i, line in enumerate(lines):
        if ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        elif in_asm:
            asm_line.add(i)
            m = re.match(r"\s*v_mfma\S*\s+(a\[\d+:\d+\])", line)
            if m:
                acc |= _agprs(m.group(1))
    n_mfma = n_settle = 0
    problems, open_at = [], None
    for i, line in enumerate(lines):
        s = line.strip()
        if i in asm_line:
            if re.match(r"v_mfma\S*\s+a\[", s):
                n_mfma += 1
                open_at = i if open_at is None else open_at
            elif s.startswith(SETTLE) and open_at is not None:
                n_settle += 1
                open_at = None
            continue
        if open_at is None or not s or s.startswith(";"):
            continue
        if re.match(r"^(\.LBB\w+:|s_cbranch|s_branch|s_setpc|s_endpgm)", s):
            problems.append(f"line {i}: block boundary before the settle: {s}")
            open_at = None
        elif _agprs(s) & acc:
            problems.append(f"line {i}: accumulator AGPR touched before the settle: {s}")
    if open_at is not None:
        problems.append("hand-written MFMAs not followed by a settle")
    return n_mfma, n_settle, problems


@pytest.fixture(scope="module", params=[(), ("JFA_DEBUG_SYNC",)], ids=["release", "debug_sync"])
def wide_unit(request):
    try:
        return build.device_asm("bwd_wide.hip", request.param)
    except RuntimeError as e:
        if "hipcc not found" in str(e):
            pytest.skip(str(e))
        raise


def test_hand_written_mfma_regions_are_closed(wide_unit):
    kernels = {m.group(1): m.group(2) for m in KERNEL.finditer(wide_unit)}
    # d = 192 and 256, each causal / non-causal / broadcast-Q
    assert len(kernels) == 6, sorted(kernels)
    for name, body in kernels.items():
        n_mfma, n_settle, problems = check_kernel(body)
        assert n_mfma >= 16 and n_settle >= 1, (name, n_mfma, n_settle)
        assert not problems, (name, problems)


def test_hand_written_mfmas_only_in_the_checked_kernels():
    """Only the dK/dV kernel calls them, and only its d >= 192 instantiations
    (those of the unit checked above) take that path."""
    for src in sorted(os.listdir(build.CSRC)):
        with open(os.path.join(build.CSRC, src)) as f:
            text = f.read()
        users = text.count("mfma4_acc_agpr(") + text.count("agpr_settle(")
        if src == "device_common.h":
            assert users == 2   # the definitions
        elif src == "bwd.hip":
            assert users == 2 and "static constexpr bool ACC_AGPR = D >= 192;" in text
        else:
            assert users == 0, src


SAMPLE = """\
\t;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[2:5], v[6:9], a[16:31]
\t;;#ASMEND
{between}
\t;;#ASMSTART
\ts_nop 15
\t;;#ASMEND
\tv_accvgpr_read_b32 v1, a0
"""


@pytest.mark.parametrize("between, expect", [
    ("\tv_add_f32_e32 v1, v2, v3", None),
    ("\tv_accvgpr_read_b32 v1, a3", "accumulator AGPR touched"),
    ("\tv_accvgpr_mov_b32 a200, a17", "accumulator AGPR touched"),
    ("\tv_accvgpr_write_b32 a31, 0", "accumulator AGPR touched"),
    ("\tv_accvgpr_read_b32 v1, a40", None),
    (".LBB3_7:", "block boundary"),
    ("\ts_cbranch_scc1 .LBB3_9", "block boundary"),
])
def test_checker_sees_planted_violations(between, expect):
    n_mfma, n_settle, problems = check_kernel(SAMPLE.format(between=between))
    assert n_mfma == 2
    if expect is None:
        assert not problems and n_settle == 1
    else:
        assert problems and expect in problems[0]


def test_checker_sees_a_missing_settle():
    text = SAMPLE.format(between="").replace("s_nop 15", "s_nop 3")
    _, n_settle, problems = check_kernel(text)
    assert n_settle == 0 and "hand-written MFMAs not followed by a settle" in problems
