"""Static checks of the decode kernel's generated gfx950 code (CPU only).

The decode kernel issues its MFMAs as inline asm, so the compiler neither
inserts wait states after them nor knows that their results arrive late.
These checks compile ``decode.hip`` to assembly and verify, for every
instantiation of the kernel:

* no instruction other than an MFMA reads or writes an MFMA's destination
  registers within 18 wait states of it (8-pass XDL results need fewer);
* inside the main loops, the accumulators are touched by MFMAs only;
* no register spills.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "host_offloaded_kv_amd", "csrc", "decode.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
MIN_WAIT_STATES = 18


def _regs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    return [t.rstrip(",") for t in line.split()[1:]]


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "decode.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(SRC), "-x", "hip",
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    found = {}
    for name in re.findall(r"^(_Z\w*decode_ws\w*):", text, re.M):
        body = text.split(f"\n{name}:", 1)[1].split(".Lfunc_end", 1)[0]
        found[name] = body.split("\n")
    assert len(found) >= 3, "expected the 16-, 32- and 64-head instantiations"
    return found


def test_no_early_reads_of_mfma_results(kernels):
    for name, lines in kernels.items():
        ins = [l.strip() for l in lines if l.strip() and not l.strip().startswith((";", "."))]
        for i, l in enumerate(ins):
            if not l.startswith("v_mfma"):
                continue
            dst = _regs(_operands(l)[0])
            waits = 0
            for x in ins[i + 1:i + 80]:
                if x.startswith("s_nop"):
                    waits += int(x.split()[1]) + 1
                    continue
                if x.startswith("v_mfma"):
                    waits += 1
                    continue
                used = set()
                for t in re.findall(r"v\[\d+:\d+\]|v\d+", " ".join(_operands(x))):
                    used |= _regs(t)
                if used & dst:
                    assert waits >= MIN_WAIT_STATES, f"{name}: '{x}' {waits} wait states after '{l}'"
                    break
                waits += 1
                if waits >= MIN_WAIT_STATES:
                    break


def test_accumulators_untouched_inside_loops(kernels):
    """Registers that an MFMA accumulates into across loop iterations (srcC
    = dst and never restarted from 0 inside the loop) are touched by MFMAs
    only, anywhere in that loop (loops nested in it -- the hand-off waits --
    included)."""
    for name, lines in kernels.items():
        headers = [i for i, l in enumerate(lines) if "Loop Header: Depth=" in l]
        assert headers, f"{name}: no loops found"
        checked = 0
        for h in headers:
            # the header's block label is the nearest label at or above the
            # annotation (nested headers carry several comment lines)
            at = next((i for i in range(h, -1, -1) if lines[i].startswith(".LBB")), None)
            assert at is not None, f"{name}: unexpected loop header layout"
            label = lines[at].split(":")[0].strip().lstrip(".")
            tag = f"Header={label[1:]} "
            member = [i for i, l in enumerate(lines) if tag in l + " "]
            first = min(member + [h])
            last = max(member + [h])
            end = next((i for i in range(last + 1, len(lines)) if lines[i].startswith((".LBB", "; %bb."))),
                       len(lines))
            body = [l.strip() for l in lines[first:end]]
            acc, restarted = set(), set()
            for l in body:
                if l.startswith("v_mfma"):
                    ops = _operands(l)
                    if ops[-1] == ops[0]:
                        acc |= _regs(ops[0])
                    elif ops[-1] == "0":
                        restarted |= _regs(ops[0])
            acc -= restarted
            if not acc:
                continue
            checked += 1
            for l in body:
                if not l or l.startswith((";", ".", "v_mfma", "s_")):
                    continue
                used = set()
                for t in re.findall(r"v\[\d+:\d+\]|v\d+", " ".join(_operands(l))):
                    used |= _regs(t)
                assert not (used & acc), f"{name}: '{l}' touches an accumulator inside a loop"
        assert checked, f"{name}: no loop accumulates through MFMAs"


def test_no_spills(kernels):
    for name, lines in kernels.items():
        assert not any("scratch_" in l for l in lines), f"{name} spills registers"
