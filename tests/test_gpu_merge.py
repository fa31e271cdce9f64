"""GPU parity of the two merge kernels of the decode step.

The library merges a segment's partials with the narrow kernel (up to 16
partial outputs per round trip) unless the launched work groups exceed 12 per
(entry, head group) segment, where the wide kernel takes 64 groups per trip.
Both are checked against the CPU oracle on each side of that rule (72 and 73
groups over 6 segments), and the wide one where a segment's 128 partials need
two of its batches (one row at its last position, every resident group
holding one tile).  Bar as elsewhere: V store and untouched bytes bit-exact,
K store within one ulp, outputs within max-abs 2e-2 and RMS 4e-3.
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def _run(A, pos, waves, seed):
    # Llama-like heads: Hkv = 8, G = 4, four kv heads per group -> 2 segments per entry
    cfg = workloads.config("tiny", A=A, S=A + 2, C=4096, Hq=32, Hkv=8, D=128, base=5.0e5,
                           seed=seed, rows="subset")
    inp = workloads.draw_decode(cfg, device="cpu")
    inp["positions"] = np.asarray(pos, dtype=np.int32)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0, waves=waves)
    assert int(run.status.item()) == 0
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


@pytest.mark.parametrize("groups", [72, 73], ids=["narrow", "wide"])
def test_merge_rule_boundary(groups):
    """3 entries x 2 segments (410 tiles): 72 groups of four waves stay with the
    narrow merge, 73 take the wide one."""
    H.log(f"merge boundary: A=3, groups={groups}")
    _run(3, [2047, 1500, 3001], 4 * groups, seed=81)


def test_wide_merge_two_batches():
    """One row at position 4095: 256 tiles over the resident groups, 128 partials per head."""
    H.log("wide merge, fan-in 128")
    _run(1, [4095], 0, seed=82)
