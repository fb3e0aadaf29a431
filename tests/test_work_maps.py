"""Host checks of the workgroup -> work-item maps the kernels use.

The maps live in the kernels' device header as host-callable functions; this
test compiles a tiny host program against that header (hipcc, host code only,
no GPU) and checks, for many grid sizes:
  * xcd_contiguous_id is a permutation of [0, grid) (every Q tile, pair or
    split-KV slice is computed exactly once), and each XCD (wg % 8) receives
    one contiguous range of logical ids;
  * dealt_id is a permutation for every grid the host selects it for (whole
    heads per XCD), and, under the placement it is built for (local
    workgroup L of an XCD on CU L mod 32, one round), every CU's Q tiles add
    up to the same number of K/V tiles to within one tile's weight per round.
"""
import os
import subprocess
import tempfile

import pytest

from exact_tiled_attention_30_amd import build

PROG = r"""
#include <cstdio>
#include "fa2_device.hpp"
int main() {
  const int big[] = {1024, 1031, 2048, 4096, 4099, 8192};
  for (int g = 1; g <= 706; ++g) {
    const int grid = g <= 700 ? g : big[g - 701];
    for (int wg = 0; wg < grid; ++wg) std::printf("x %d %d %d\n", grid, wg, fa2::xcd_contiguous_id(wg, grid));
  }
  const int nqs[] = {1, 2, 4, 8, 16, 32};
  for (int nq : nqs)
    for (int heads_per_xcd = 1; heads_per_xcd * nq <= 512; ++heads_per_xcd) {
      const int grid = 8 * heads_per_xcd * nq;
      for (int wg = 0; wg < grid; ++wg)
        std::printf("d %d %d %d %d\n", grid, nq, wg, fa2::dealt_id(wg, grid, nq));
    }
  return 0;
}
"""


@pytest.fixture(scope="module")
def maps():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "maps.hip")
        exe = os.path.join(tmp, "maps")
        with open(src, "w") as f:
            f.write(PROG)
        subprocess.run([build.hipcc(), "--cuda-host-only", "-O1", "-std=c++17", "-I", build.CSRC,
                        src, "-o", exe], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    xs, ds = {}, {}
    for line in out.splitlines():
        p = line.split()
        if p[0] == "x":
            xs.setdefault(int(p[1]), []).append((int(p[2]), int(p[3])))
        else:
            ds.setdefault((int(p[1]), int(p[2])), []).append((int(p[3]), int(p[4])))
    return xs, ds


def test_xcd_contiguous_id_is_a_permutation_with_contiguous_xcd_ranges(maps):
    xs, _ = maps
    assert len(xs) == 706
    for grid, pairs in xs.items():
        ids = [i for _, i in pairs]
        assert sorted(ids) == list(range(grid)), grid
        for xcd in range(8):
            mine = sorted(i for wg, i in pairs if wg % 8 == xcd)
            assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True, (grid, xcd)
            # consecutive hardware slots of one XCD walk its range in order
            slots = [i for wg, i in sorted(pairs) if wg % 8 == xcd]
            assert slots == sorted(slots), (grid, xcd)


def test_dealt_id_is_a_permutation_and_balances_cus(maps):
    _, ds = maps
    assert ds
    for (grid, nq), pairs in ds.items():
        ids = [i for _, i in pairs]
        assert sorted(ids) == list(range(grid)), (grid, nq)
        per = grid // 8
        for xcd in range(8):
            # whole heads per XCD: the XCD's ids are exactly its own heads' tiles
            mine = sorted(i for wg, i in pairs if wg % 8 == xcd)
            assert mine == list(range(xcd * per, (xcd + 1) * per)), (grid, nq, xcd)
            # weight of item t of a head: the kernel runs Q tile nq-1-t, which
            # streams nq-t K/V tile rows (of the Q tile's height); CU of a
            # workgroup: its local index on the XCD mod 32
            totals = {}
            for wg, i in pairs:
                if wg % 8 == xcd:
                    cu = (wg // 8) % 32
                    totals[cu] = totals.get(cu, 0) + (nq - i % nq)
            if per % 64 == 0:
                # an even number of full rounds: snake order pairs every CU's
                # heavy and light ranks, so all CUs carry the same total
                assert max(totals.values()) == min(totals.values()), (grid, nq, xcd, totals)
            else:
                assert max(totals.values()) - min(totals.values()) <= nq, (grid, nq, xcd)
