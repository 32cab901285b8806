"""The GELU table the HIP library builds at compile time (csrc/gelu_table.h,
the same constexpr code compiled here by the host compiler) against the
oracle's GELU, entry by entry: every slot of both signs over |y| in
[2^-14, 128), the sentinel slots, and the zero padding.  The oracle's own
GELU is pinned to a 90-digit evaluation in test_oracle_gelu.py."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_compile_time_gelu_table_matches_oracle(tmp_path):
    exe = str(tmp_path / "gelu_table_dump")
    r = subprocess.run(["g++", "-std=c++20", "-O1", "-fconstexpr-ops-limit=1000000000",
                        os.path.join(HERE, "gelu_table_dump.cpp"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    e_lo, stride, n = (int(v) for v in out[:3])
    tab = np.array([int(v, 16) for v in out[3:]], np.uint16)
    assert len(tab) >= n and np.all(tab[n:] == 0)
    span = stride - 1
    assert span == 21 * 128 and n == 2 * stride
    j = np.arange(span)
    mags = ((e_lo << 7) + j).astype(np.uint16)
    for sgn, base in ((0, 0), (0x8000, stride)):
        x = (mags | sgn).astype(np.uint16)
        ref = oracle.gelu_tanh_bf16(x)
        got = tab[base:base + span]
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"sign {sgn:#x}: {bad.size} entries differ, first at magnitude {mags[bad[0]]:#06x}"
        assert tab[base + span] == 0x7FFF                      # the sentinel slot
    # the upper end of the table holds the |y| >= 32 rule exactly: y and -0
    big = mags >= 0x4200
    assert np.all(tab[:span][big] == mags[big]) and np.all(tab[stride:stride + span][big] == 0x8000)
