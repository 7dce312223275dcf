"""Checks on the gfx950 assembly of the flash and projection kernels (CPU
only: hipcc cross-compiles, nothing runs).

* The K/V (and projection operand) tile DMA is issued from inline asm that
  loads M0 itself.  The asm
  declares M0 clobbered, which the compiler may not honour for a reserved
  register, so the asm is only safe while no compiler-generated instruction
  keeps a value in M0.  The test requires every M0 reference in the device
  code to be one of the asm's own two instructions.
* The bf16 kernels run without a private (scratch) segment: no spill, so
  no scratch memory for the runtime to provide, and none in the main loop,
  where a spill would cost a memory round trip per step.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "alternating_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(tmp_path_factory, name):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / (name + ".s"))
    cmd = [HIPCC, "-x", "hip", "-S", "--cuda-device-only", "-O3", "-std=c++17",
           "--offload-arch=gfx950", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, name), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, "flash_attn.hip")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "proj_gemm.hip")


def _kernels(text):
    """name -> (body, private segment bytes) for each kernel in the file."""
    res = {}
    for m in re.finditer(r"^(_Z\w+):\s*(?:;.*)?$", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.end())
        seg = re.search(r"\.amdhsa_kernel " + re.escape(name) +
                        r".*?\.amdhsa_private_segment_fixed_size (\d+)", text, re.S)
        res[name] = (text[m.end():end], int(seg.group(1)) if seg else None)
    return res


def _instructions(body):
    for line in body.split("\n"):
        t = line.strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            yield t.split(";")[0].strip()


def _check_m0(text):
    users = [i for i in _instructions(text) if re.search(r"\bm0\b", i)]
    assert users, "the tile DMA no longer sets M0"
    for ins in users:
        op = ins.split()[0]
        assert op == "global_load_lds_dwordx4" or re.fullmatch(r"s_mov_b32 m0, s\d+", ins), ins


def test_m0_only_in_the_dma_asm(asm, gemm_asm):
    _check_m0(asm)
    _check_m0(gemm_asm)


def _main_loop(body):
    """The longest loop (label .. its back-branch) that holds MFMAs."""
    lines = body.split("\n")
    labels = {l.split(":")[0]: i for i, l in enumerate(lines) if re.match(r"^\.LBB\d+_\d+:", l)}
    best = []
    for i, l in enumerate(lines):
        m = re.search(r"s_c?branch\w*\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            seg = lines[labels[m.group(1)]:i + 1]
            if sum("v_mfma" in x for x in seg) and len(seg) > len(best):
                best = seg
    return best


def test_projection_kernel_spill_free(gemm_asm):
    ks = {n: v for n, v in _kernels(gemm_asm).items() if "linear_bf16_kernel" in n}
    assert len(ks) == 1
    for name, (body, private) in ks.items():
        assert sum("v_mfma" in x for x in _main_loop(body)) >= 32, name
        assert private == 0, (name, private)


def test_bf16_kernels_spill_free(asm):
    ks = {n: v for n, v in _kernels(asm).items() if "flash_bf16_kernel" in n}
    assert len(ks) == 3
    for name, (body, private) in ks.items():
        loop = _main_loop(body)
        assert sum("v_mfma" in x for x in loop) >= 64, name
        assert not [x for x in loop if "scratch_" in x], name
        assert private == 0, (name, private)
