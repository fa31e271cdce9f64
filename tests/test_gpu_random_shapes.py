"""GPU parity on seeded random shapes: combinations the fixed cases do not
cover, each drawn within the limits include/mllm.h documents and checked in
full against the CPU oracle.

Decode: batch size, slot count, kv heads (1, 2, 4, 8, 16), query heads per kv
head (1 to 16), head dim (64, 128), storage type, capacity, positions (mixing
0, tile edges and the last position of a row) and the wave count.  Chunk
prefill: batch size, chunk width T, heads, head dim, storage type, and per-entry
starts and lengths (a fresh prompt, one token, the whole chunk, ragged).

Bar as elsewhere: V store and untouched bytes bit-exact, K store within one
ulp, outputs within max-abs 2e-2 and RMS 4e-3.
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


def _decode_case(seed):
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8, 16]))
    G = int(rng.integers(1, 17))
    D = int(rng.choice([64, 128]))
    A = int(rng.integers(1, 41))
    S = A + int(rng.integers(0, 5))
    Cap = int(rng.choice([33, 64, 130, 257, 600]))
    dtype = str(rng.choice(["bf16", "f16"]))
    # positions: a mix of 0, tile edges, the row's last position and uniform draws
    special = [0, 1, 15, 16, 31, 32, 33, 63, 64, Cap - 1]
    pos = np.where(rng.random(A) < 0.4, rng.choice(special, A), rng.integers(0, Cap, A))
    pos = np.minimum(pos, Cap - 1).astype(np.int32)
    waves = int(rng.choice([0, 0, 1, 3, 7, 64]))
    return dict(A=A, S=S, Cap=Cap, Hq=Hkv * G, Hkv=Hkv, D=D, dtype=dtype, pos=pos, waves=waves)


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    c = _decode_case(seed)
    H.log(f"random decode {seed}: A={c['A']} S={c['S']} C={c['Cap']} Hq={c['Hq']} "
          f"Hkv={c['Hkv']} D={c['D']} {c['dtype']} waves={c['waves']}")
    cfg = workloads.config("tiny", A=c["A"], S=c["S"], C=c["Cap"], Hq=c["Hq"], Hkv=c["Hkv"],
                           D=c["D"], seed=2000 + seed, rows="subset", dtype=c["dtype"])
    inp = workloads.draw_decode(cfg, device="cpu")
    inp["positions"] = c["pos"]
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0, waves=c["waves"])
    assert int(run.status.item()) == 0
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


def _chunk_case(seed):
    rng = np.random.default_rng(3000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 9))
    D = int(rng.choice([64, 128]))
    A = int(rng.integers(1, 7))
    T = int(rng.choice([1, 2, 31, 64, 65, 100, 128, 129, 257]))
    dtype = str(rng.choice(["bf16", "f16"]))
    lens = np.where(rng.random(A) < 0.3, rng.choice([1, T], A), rng.integers(1, T + 1, A))
    starts = np.where(rng.random(A) < 0.3, rng.choice([0, 63, 64, 127], A),
                      rng.integers(0, 400, A))
    rows = rng.permutation(A + 2)[:A]
    return dict(A=A, T=T, Hq=Hkv * G, Hkv=Hkv, D=D, dtype=dtype, lens=lens.astype(np.int32),
                starts=starts.astype(np.int32), rows=rows.astype(np.int32))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
def test_random_chunk(kernel, seed):
    c = _chunk_case(seed)
    H.log(f"random chunk {seed} kernel={kernel}: A={c['A']} T={c['T']} Hq={c['Hq']} "
          f"Hkv={c['Hkv']} D={c['D']} {c['dtype']} starts={c['starts'].tolist()} "
          f"lens={c['lens'].tolist()}")
    Cap = int((c["starts"] + c["lens"]).max()) + 5
    cfg = workloads.config("prefill", A=c["A"], S=c["A"] + 2, C=Cap, T=c["T"], Hq=c["Hq"],
                           Hkv=c["Hkv"], D=c["D"], base=1.0e4, seed=4000 + seed,
                           dtype=c["dtype"])
    run = C.ChunkRun(cfg, c["starts"], c["lens"], c["rows"])
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(kernel)
    C.parity(run, Kpre, Vpre)
    C.untouched(run, Kpre, Vpre)
