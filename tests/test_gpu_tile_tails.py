"""Parity on planted expert row counts: every residue class of an expert's
last M-tile that the grouped GEMM treats differently.

The expert GEMM deals the 16-row MFMA fragments of a tile to its wavefront
rows in turn and skips the fragments past the expert's last row, so the
counts below put an expert's last tile at 1, 15, 16, 17, 63, 64, 65, 127 ...
rows for each kernel shape (32-, 128- and 256-row M-tiles, chosen from the
average rows per expert).  Routing is planted: W_gate reads the first E
features of x, and each token's own expert gets a feature of 16 against
N(0, 1) noise, so the choice is never near a tie and the kept counts are
exactly the planted ones.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, Run, check_layer, say
from workloads import Workload

pytestmark = pytest.mark.gpu

TAIL_CASES = {
    # average 35.6 rows per expert: 32-row tiles
    "short_tiles": ((1, 15, 16, 17, 31, 32, 33, 47, 64, 100), 0),
    # average 90: 256-row tiles, one per expert up to 255 rows
    "wide_tiles": ((1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200, 255), 0),
    # average 458: 128-row tiles; T = 3665 also leaves a short last tile in
    # the shared expert's GEMMs over all tokens
    "long_tiles_shared": ((385, 400, 447, 448, 449, 511, 512, 513), 1),
}


def _plant(run: Run, counts, seed=11):
    """Overwrite x and W_gate (device and host copies) so that token t picks
    expert owner[t], with owner a shuffled list holding counts[e] copies of
    e."""
    w = run.w
    owner = np.repeat(np.arange(w.E), counts)
    np.random.default_rng(seed).shuffle(owner)
    x = run.hx.clone()
    x[torch.arange(w.T), torch.from_numpy(owner)] = 16.0
    Wg = torch.zeros((w.d, w.E), dtype=run.hWg.dtype)
    Wg[torch.arange(w.E), torch.arange(w.E)] = 1.0
    run.hx, run.hWg = x, Wg
    run.x, run.Wg = x.to(DEV), Wg.to(DEV)
    return owner


@pytest.mark.parametrize("case", sorted(TAIL_CASES))
def test_forward_planted_tile_tails(case):
    counts, S = TAIL_CASES[case]
    w = Workload(f"tails_{case}", T=int(sum(counts)), d=192, F=320, E=len(counts), k=1,
                 S=S, capacity_factor=0.0)
    say(f"[tails] {case}: counts {counts}")
    run = Run(w)
    _plant(run, counts)
    e = check_layer(run, f"tails_{case}")
    assert e["dropped"] == 0
    st = run.forward(stats=True)[1]
    assert np.array_equal(st["kept"], np.asarray(counts))
