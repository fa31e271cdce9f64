"""GPU parity of the FP16 storage type against the CPU oracle (the same kernels,
instantiated for FP16, through the C ABI).

Bar, as for BF16: V store and every untouched cache byte bit-exact, rotated K
store within one FP16 ulp, output within max-abs 2e-2 and RMS 4e-3 over the
whole output.  The oracle runs with FP16 storage (IEEE binary16 conversions).
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import test_gpu_chunk as C
import test_gpu_prefill as P
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def small_case(D, Hq, Hkv, positions, Cap, seed=0, inactive="normal"):
    A = len(positions)
    cfg = workloads.config("tiny", A=A, S=A + 3, C=Cap, Hq=Hq, Hkv=Hkv, D=D, seed=seed,
                           inactive=inactive, dtype="f16")
    inp = workloads.draw_decode(cfg, device="cpu")
    inp["positions"] = np.asarray(positions, dtype=np.int32)
    return cfg, inp


@pytest.mark.parametrize("kernel", [0, 1], ids=["tuned", "readable"])
@pytest.mark.parametrize("mirror", [True, False], ids=["mirror", "nomirror"])
def test_f16_tiny_parity(kernel, mirror):
    cfg = workloads.config("tiny", dtype="f16")
    H.log(f"f16 tiny kernel={kernel} mirror={mirror}")
    inp = workloads.draw_decode(cfg, device="cpu")
    assert inp["q"].dtype == torch.float16
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=kernel, mirror=mirror)
    assert int(run.status.item()) == 0
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


EDGE_POS = [0, 1, 15, 16, 31, 32, 33, 63, 64, 65, 127, 128, 255, 256, 257, 511, 639]
HEADS = [(4, 4), (4, 2), (8, 2), (16, 2), (32, 2), (6, 2)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", HEADS, ids=[f"{q}x{k}" for q, k in HEADS])
@pytest.mark.parametrize("waves", [5, 0], ids=["w5", "wdev"])
def test_f16_edge_positions(D, heads, waves):
    """Every tile boundary and every query-group width (1 to 16 query heads per
    kv head) of the FP16 decode kernel."""
    Hq, Hkv = heads
    H.log(f"f16 edge D={D} Hq={Hq} Hkv={Hkv} waves={waves}")
    cfg, inp = small_case(D, Hq, Hkv, EDGE_POS, Cap=640, seed=D + Hq + waves)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0, waves=waves)
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


@pytest.mark.parametrize("name", ["llama3_8b", "ragged"])
def test_f16_full_config_parity(name):
    cfg = workloads.config(name, dtype="f16")
    H.log(f"f16 full config {name}: generating on device")
    inp = workloads.draw_decode(cfg, device="cuda")
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    H.log(f"f16 full config {name}: running")
    run.run()
    H.log(f"f16 full config {name}: oracle on every entry")
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))
    assert torch.isfinite(run.out.float()).all()


PREFILL_SHAPES = [(17, 8, 2, 128), (65, 8, 2, 64), (129, 8, 2, 128), (200, 6, 2, 64)]


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
@pytest.mark.parametrize("shape", PREFILL_SHAPES,
                         ids=[f"T{t}_{q}x{k}_D{d}" for t, q, k, d in PREFILL_SHAPES])
def test_f16_prefill_shapes(kernel, shape):
    T, Hq, Hkv, D = shape
    H.log(f"f16 prefill kernel={kernel} T={T} Hq={Hq} Hkv={Hkv} D={D}")
    cfg = workloads.config("prefill", A=3, S=5, C=max(T + 7, 64), T=T, Hq=Hq, Hkv=Hkv, D=D,
                           base=1.0e4, seed=T + Hq, rows_override=[4, 0, 2], dtype="f16")
    run = P.PrefillRun(cfg)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(kernel)
    assert torch.isfinite(run.out.float()).all()
    P.parity(run, Kpre, Vpre)
    P.untouched(run, Kpre, Vpre)


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
@pytest.mark.parametrize("case", C.CASES[1:6:2], ids=[f"T{c[0]}_{c[1]}x{c[2]}_D{c[3]}"
                                                      for c in C.CASES[1:6:2]])
def test_f16_chunk_cases(kernel, case):
    T, Hq, Hkv, D, starts, lens = case
    H.log(f"f16 chunk kernel={kernel} T={T} Hq={Hq} Hkv={Hkv} D={D} starts={starts} lens={lens}")
    cfg = C._case_cfg(T, Hq, Hkv, D, starts, lens, seed=T + 3 * Hq)
    cfg["dtype"] = "f16"
    rows = [5, 0, 3, 1]
    run = C.ChunkRun(cfg, starts, lens, rows)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(kernel)
    C.parity(run, Kpre, Vpre)
    C.untouched(run, Kpre, Vpre)


def test_f16_full_prefill():
    """16 prompts x 1024 tokens in FP16, 32/8/128: sampled outputs of two rows
    against the oracle, every store of those rows, the rest untouched."""
    cfg = workloads.config("prefill", dtype="f16")
    H.log("f16 prefill full config: generating")
    run = P.PrefillRun(cfg)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    assert torch.isfinite(run.out.float()).all()
    t_list = [0, 1, 63, 64, 127, 128, 129, 511, 512, 1000, 1023]
    P.parity(run, Kpre, Vpre, entries=[3, 12], t_list=t_list)
    P.untouched(run, Kpre, Vpre)
