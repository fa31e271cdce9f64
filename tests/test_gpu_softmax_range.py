"""GPU parity where the scores span a wide range along the sequence, so the
online softmax's running maximum keeps growing past its headroom (the kernels
rescale their partial sums tile after tile) or starts at its peak and later
weights underflow to zero.

The keys of position j (prior cache contents and the new tokens alike) are
scaled by c_j before the call: growing rows use c_j = 1 + j / 4 (the maximum
score of a 32-key tile exceeds the previous tiles' by far more than the
kernels' headroom), shrinking rows c_j = 1 + (L - j) / 4.  Expected values
come from the CPU oracle on the same inputs; the bar is the usual one.
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import test_gpu_chunk as C
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def _scales(n, grow):
    j = np.arange(n, dtype=np.float64)
    return 1.0 + (j if grow else (n - 1 - j)) / 4.0


def _scaled(x, c):
    """x [..., L, H, D] (positions on dim -3) times c [L], rounded to the storage type."""
    f = x.float() * torch.as_tensor(c, dtype=torch.float32, device=x.device)[:, None, None]
    return f.to(x.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D,G", [(64, 4), (128, 4), (128, 8), (64, 16)])
def test_decode_growing_and_shrinking_scores(dtype, D, G):
    """G <= 4 carries the BF16 query exactly in three parts, larger groups in two."""
    A, Cap = 6, 600
    H.log(f"decode score range D={D} G={G} {dtype}")
    cfg = workloads.config("tiny", A=A, S=A + 1, C=Cap, Hq=2 * G, Hkv=2, D=D, seed=61 + D + G,
                           rows="subset", dtype=dtype)
    inp = workloads.draw_decode(cfg, device="cpu")
    pos = np.array([599, 300, 257, 64, 500, 33], dtype=np.int32)
    inp["positions"] = pos
    for a in range(A):
        r, p = int(inp["rows"][a]), int(pos[a])
        c = _scales(p + 1, grow=a % 2 == 0)
        # FP16 keeps the largest products finite: c stays below 151, |k| below ~700
        inp["Kc"][r, :p + 1] = _scaled(inp["Kc"][r, :p + 1], c)
        inp["k_new"][a] = _scaled(inp["k_new"][a:a + 1], c[p:p + 1])[0]
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    for kernel in (0, 1):
        run.Kc.copy_(Kpre)
        run.Vc.copy_(Vpre)
        run.run(kernel=kernel)
        assert int(run.status.item()) == 0
        H.full_parity(run, Kpre, Vpre)
        H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
def test_chunk_growing_and_shrinking_scores(kernel, dtype):
    T, Hq, Hkv, D = 200, 8, 2, 128
    starts = np.array([0, 130, 64, 251], dtype=np.int32)
    lens = np.array([200, 200, 97, 150], dtype=np.int32)
    rows = np.array([3, 0, 4, 1], dtype=np.int32)
    H.log(f"chunk score range kernel={kernel} {dtype}")
    Cap = int((starts + lens).max()) + 3
    cfg = workloads.config("prefill", A=4, S=5, C=Cap, T=T, Hq=Hq, Hkv=Hkv, D=D, base=1.0e4,
                           seed=71, dtype=dtype)
    run = C.ChunkRun(cfg, starts, lens, rows)
    for a in range(4):
        s, n, r = int(starts[a]), int(lens[a]), int(rows[a])
        c = _scales(s + n, grow=a % 2 == 0)
        run.Kc[r, :s] = _scaled(run.Kc[r, :s], c[:s])
        run.k[a, :n] = _scaled(run.k[a, :n], c[s:s + n])
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(kernel)
    C.parity(run, Kpre, Vpre)
    C.untouched(run, Kpre, Vpre)
