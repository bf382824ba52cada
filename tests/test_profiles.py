"""CPU checks of the committed profiler summaries: every library kernel a
summary names exists in the built library (a summary taken from an older
build whose kernels were since renamed fails here), every summary gives the
rocprofv3 command that made it over a committed entry point, and the kernel
the benchmark's roofline times is one of them."""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "query_aware_prefill_amd", "libquail.so")
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")) +
                   glob.glob(os.path.join(ROOT, "profiles", "*.txt")))


def _kernel_names():
    if shutil.which("nm") is None:
        pytest.skip("nm is not available")
    out = subprocess.run(["nm", "-C", LIB], capture_output=True, text=True, check=True).stdout
    names = set()
    for line in out.splitlines():
        m = re.search(r"(quail::(?!__device_stub__)\w+(?:<[^()]*>)?)\(", line)
        if m:
            names.add(m.group(1))
    return names


def _named(text):
    """quail:: kernels a summary names (template arguments kept, parameters
    dropped); names cut short with '...' are skipped."""
    out = set()
    for m in re.finditer(r"quail::\w+(?:<[^()`|]*>)?", text):
        s = m.group(0)
        if s.endswith("...") or "<" in s and not s.endswith(">"):
            continue
        if re.match(r"quail::\w+_kernel", s):
            out.add(s)
    return out


def test_every_summary_names_existing_kernels_and_its_command():
    assert SUMMARIES
    have = _kernel_names()
    assert "quail::attn_direct_kernel<4, false, false, 0, false>" in have
    for path in SUMMARIES:
        text = open(path).read()
        missing = sorted(n for n in _named(text) if n not in have)
        assert not missing, (os.path.basename(path), missing)
        assert "rocprofv3" in text and ("bench.py" in text), os.path.basename(path)


def test_roofline_kernel_is_in_the_library():
    src = open(os.path.join(ROOT, "bench.py")).read()
    names = re.findall(r'"(quail::(?:attn|gemm)_direct_kernel<[^"]*>)"', src)
    assert names
    have = _kernel_names()
    for n in names:
        assert n in have, n
