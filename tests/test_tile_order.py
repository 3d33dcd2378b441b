"""The workgroup -> (query tile, head) schedule of the attention kernels (no GPU).

Compiles a host program around the kernels' own `tile_of` (csrc/common.h) and checks,
over many grid shapes, that every (tile, head) is computed exactly once, that the
tile-major order runs the heaviest tiles first, and that the banded order keeps the
query heads of a K/V head on one XCD (workgroup index mod 8) in bands of one head,
heaviest band first.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from fp8_causal_prefill_tiled_amd import build

PROG = r"""
#include "common.h"
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
    const int BH = std::atoi(argv[1]), ratio = std::atoi(argv[2]), nt = std::atoi(argv[3]);
    for (int L = 0; L < BH * nt; ++L) {
        int tile, bh;
        attnfwd::tile_of(L, BH, ratio, nt, tile, bh);
        std::printf("%d %d\n", tile, bh);
    }
    return 0;
}
"""

# (query heads in all = B * Hq, query heads per K/V head, query tiles)
SHAPES = [(8, 1, 1), (32, 1, 128), (32, 4, 64), (16, 1, 128), (40, 5, 2), (48, 1, 1), (64, 4, 2),
          (64, 8, 33), (64, 1, 32), (128, 1, 64), (256, 4, 32), (2048, 1, 16), (64, 32, 5), (24, 3, 9),
          (96, 12, 70), (64, 2, 31)]


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("tile_order")
    src = d / "tile_order.cpp"
    src.write_text(PROG)
    exe = d / "tile_order"
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-I", build.CSRC, str(src),
                    "-o", str(exe)], check=True, capture_output=True)
    return str(exe)


def schedule(prog, BH, ratio, nt):
    out = subprocess.run([prog, str(BH), str(ratio), str(nt)], check=True, capture_output=True, text=True).stdout
    return np.array([[int(x) for x in line.split()] for line in out.splitlines()])


@pytest.mark.parametrize("BH,ratio,nt", SHAPES)
def test_every_tile_once(prog, BH, ratio, nt):
    s = schedule(prog, BH, ratio, nt)
    assert s.shape == (BH * nt, 2)
    assert (s[:, 0] >= 0).all() and (s[:, 0] < nt).all() and (s[:, 1] >= 0).all() and (s[:, 1] < BH).all()
    assert len({(t, b) for t, b in s}) == BH * nt


@pytest.mark.parametrize("BH,ratio,nt", SHAPES)
def test_order(prog, BH, ratio, nt):
    s = schedule(prog, BH, ratio, nt)
    L = np.arange(BH * nt)
    banded = BH > 32 and (BH // ratio) % 8 == 0
    if not banded:
        # tile-major, heaviest (highest) tile first
        assert (s[:, 0] == nt - 1 - L // BH).all() and (s[:, 1] == L % BH).all()
        return
    xcd = L % 8
    # every K/V head (ratio consecutive query heads) is read through one XCD
    for g in range(BH // ratio):
        assert len(set(xcd[s[:, 1] // ratio == g])) == 1
    # per XCD: bands of up to 32 tiles of one query head, heaviest band first
    G, nh = 32, BH // 8
    for x in range(8):
        sx = s[xcd == x]
        assert len(sx) == nh * nt
        band = (nt - 1 - sx[:, 0]) // G
        assert (np.diff(band) >= 0).all()
        # within a band, each query head's tiles are consecutive
        for b in np.unique(band):
            heads = sx[band == b][:, 1]
            changes = np.count_nonzero(np.diff(heads))
            assert changes == nh - 1
