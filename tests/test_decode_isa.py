"""Checks on the gfx950 assembly of the decode kernels (CPU only: hipcc
cross-compiles).

The score chain is written as inline-asm MFMAs with the accumulator in
VGPRs, so the compiler does not know that an MFMA's result lands some 30
cycles after it issues.  If register allocation ever inserts a copy (or any
other access) of the accumulator between two chain MFMAs, that instruction
reads a sum still in flight and silently drops K-steps from the scores.
This test compiles the kernels and requires every score chain to be 36
MFMAs on one accumulator with nothing else touching those registers in
between."""
import os
import re
import subprocess
import tempfile

import pytest

from sparse_mla_amd import build

CHAIN_LEN = 36  # 512 latent + 64 rotary features, 16 per MFMA


def _vgprs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def chain_violations(asm: str):
    """(number of chains found, list of violations) over the decode kernels."""
    problems, chains = [], 0
    for fn in re.findall(r"^(_Z\w*decode_kernel\w*):", asm, re.M):
        start = asm.index(fn + ":")
        end = asm.index(".Lfunc_end", start)
        lines = [l.strip() for l in asm[start:end].splitlines()]
        lines = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
        i = 0
        while i < len(lines):
            t = lines[i].replace(",", " ").split()
            # A chain starts with a VGPR-accumulator MFMA whose C operand is 0.
            if t[0] == "v_mfma_f32_32x32x16_bf16" and t[1].startswith("v[") and t[4] == "0":
                acc = _vgprs(t[1])
                n, j = 1, i + 1
                while n < CHAIN_LEN and j < len(lines):
                    u = lines[j].replace(",", " ").split()
                    if u[0] == "v_mfma_f32_32x32x16_bf16" and _vgprs(u[1]) == acc:
                        if _vgprs(u[4]) != acc:
                            problems.append(f"{fn}: chain MFMA accumulates another register: {lines[j]}")
                        n += 1
                    else:
                        touched = set().union(*[_vgprs(tok) for tok in u[1:]]) if len(u) > 1 else set()
                        if touched & acc:
                            problems.append(f"{fn}: '{lines[j]}' touches the accumulator after MFMA {n}")
                    j += 1
                if n != CHAIN_LEN:
                    problems.append(f"{fn}: chain of {n} MFMAs")
                chains += 1
                i = j
            else:
                i += 1
    return chains, problems


@pytest.fixture(scope="module")
def decode_asm():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build.HIPCC] + flags + ["--cuda-device-only", "-S", "-o", out, build.SOURCES[0]]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return open(out).read()


def test_score_chains_untouched(decode_asm):
    chains, problems = chain_violations(decode_asm)
    # 4 kernels (dense/sparse x one split/several), each with at least the
    # first block's chain and the loop's chain.
    assert chains >= 8
    assert not problems, "\n".join(problems[:10])


def test_checker_catches_a_mid_chain_copy():
    """The checker itself: a copy of the accumulator between chain MFMAs."""
    mfma = "v_mfma_f32_32x32x16_bf16"
    body = [f"\t{mfma} v[18:33], v[2:5], v[40:43], 0"]
    body += [f"\t{mfma} v[18:33], v[2:5], v[40:43], v[18:33]"] * 33
    body += ["\tv_mov_b64_e32 v[50:51], v[18:19]"]
    body += [f"\t{mfma} v[18:33], v[2:5], v[40:43], v[18:33]"] * 2
    asm = "_ZN3mla12decode_kernelE:\n" + "\n".join(body) + "\n.Lfunc_end0:\n"
    chains, problems = chain_violations(asm)
    assert chains == 1 and len(problems) == 1 and "v_mov_b64" in problems[0]
