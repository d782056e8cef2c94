"""Seeded mutation check of the container parser under AddressSanitizer and
UBSan (host only, no GPU).

`fuzz_blob_info.cpp` is built together with the library's host sources with
`-fsanitize=address,undefined`; it applies thousands of random corruptions
to a container of every layout and calls dfc_blob_info on each.  Every call
must return, an out-of-range read or undefined arithmetic aborts the run,
and every accepted container must keep its sections inside the buffer with
the sizes the decode kernels index without bounds checks."""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "lossless_entropy_coded_dfc_amd", "csrc")


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("fuzz") / "fuzz_blob_info")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "fuzz_blob_info.cpp"),
           os.path.join(CSRC, "dfc_host.cpp"), os.path.join(CSRC, "dfc_ans_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("no sanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


CASES = {
    "flat C16": lambda x: dfc.encode(x),
    "flat C4": lambda x: dfc.encode(x, chunk_bytes=4, lut_bits=8),
    "padded C8": lambda x: dfc.encode(x, chunk_bytes=8, layout=dfc.LAYOUT_PADDED),
    "panel": lambda x: dfc.encode(x, layout=dfc.LAYOUT_PANEL, panel_k=64),
    "ans 16 steps": lambda x: dfc.encode(x, layout=dfc.LAYOUT_ANS, ans_steps=16),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parser_survives_mutations(fuzzer, tmp_path, case):
    x = synth.gaussian_with_outliers((96, 320), 0.02, (140, len(case)))
    blob = CASES[case](x)
    path = tmp_path / "blob.bin"
    path.write_bytes(np.asarray(blob, dtype=np.uint8).tobytes())
    r = subprocess.run([fuzzer, str(path), "4000", str(141 + len(case))], capture_output=True, text=True,
                       timeout=600, env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    counts = json.loads(r.stdout.strip().splitlines()[-1])
    assert counts["failures"] == 0
    assert counts["rejected"] > 0 and counts["accepted"] + counts["rejected"] == 4000
