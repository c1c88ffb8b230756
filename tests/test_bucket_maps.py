"""Host checks of the select's bucket maps and order-preserving keys.

Compiles tests/bucket_maps_host.cpp against the kernels' own header
(score_top_token_amd/csrc/li_bucket.h) with the host C++ compiler and runs it:
every map stays in range and monotone for finite, infinite, equal and
inverted bounds and for values outside them; f2key orders every float
(signed zeros equal) and key2f inverts it."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "score_top_token_amd", "csrc")


def test_bucket_maps_on_host():
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "bucket_maps")
        subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-I", CSRC,
                        os.path.join(HERE, "bucket_maps_host.cpp"), "-o", exe], check=True)
        res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1].startswith("ok ")
