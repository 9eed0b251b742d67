"""Code generation of the HIP kernels for gfx950 (no GPU: hipcc emits device
assembly here). Two properties that the kernels' speed depends on and that a
small source change can silently break:

- no out-of-line device calls: a shared device function the compiler stops
  inlining is compiled with generic pointers, so its global and LDS accesses
  become flat instructions (one such call slowed the layout plan kernel by
  6 us);
- no flat memory instructions and no register spills to scratch memory.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "combine_router_topk_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# kernel -> allowed private segment bytes (none at present)
SCRATCH_ALLOWED: dict[str, int] = {}


def compile_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src)[:-4] + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "--cuda-device-only", "-S",
                    src, "-o", out], check=True, capture_output=True, timeout=300)
    return out


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    d = tempfile.mkdtemp(prefix="moe_asm_")
    try:
        with ThreadPoolExecutor(max_workers=8) as ex:
            outs = list(ex.map(lambda s: compile_asm(s, d), srcs))
        yield {os.path.basename(o): open(o).read() for o in outs}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def kernels(asm: str):
    """(kernel name, its instruction text, private segment bytes) per kernel."""
    out = []
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@\S+\n(.*?)^\.Lfunc_end", asm, re.S | re.M):
        name = m.group(1)
        body = m.group(2)
        priv = re.search(rf"\.amdhsa_kernel {re.escape(name)}\n(?:.*\n)*?\s*\.amdhsa_private_segment_fixed_size (\d+)", asm)
        out.append((name, body, int(priv.group(1)) if priv else 0))
    return out


def short(name: str) -> str:
    m = re.search(r"N_1\d+(\w+?kernel)", name) or re.search(r"(\w+kernel)", name)
    return m.group(1) if m else name


def test_every_source_compiles_to_kernels(device_asm):
    found = {f: len(kernels(a)) for f, a in device_asm.items()}
    assert all(n > 0 for f, n in found.items() if f != "abi.s"), found


def test_no_out_of_line_calls_or_flat_accesses(device_asm):
    bad = []
    for f, asm in device_asm.items():
        for name, body, _ in kernels(asm):
            if "s_swappc" in body:
                bad.append((f, short(name), "call"))
            if re.search(r"\bflat_(load|store|atomic)", body):
                bad.append((f, short(name), "flat"))
    assert not bad, bad


def test_no_unexpected_scratch(device_asm):
    bad = []
    for f, asm in device_asm.items():
        for name, _, priv in kernels(asm):
            if priv > SCRATCH_ALLOWED.get(short(name), 0):
                bad.append((f, short(name), priv))
    assert not bad, bad
