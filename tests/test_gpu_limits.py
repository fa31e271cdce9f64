"""GPU parity at sizes past the launch-grid limits of the y and z dimensions
(65535): a decode batch of 70000 entries, a prefill of 66000 tokens, and a
decode at the last position of a 131072-position row.  Outputs of sampled
entries and query positions are checked against the CPU oracle; every store
and every untouched byte is checked in full.
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import positions_aware_cached_amd as pac
import workloads
from bf16util import ulp_dist

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


@pytest.mark.parametrize("kernel", [0, 1], ids=["tuned", "readable"])
def test_decode_70000_entries(kernel):
    A, C = 70000, 40
    cfg = workloads.config("tiny", A=A, S=A, C=C, Hq=2, Hkv=1, D=64, seed=51, rows="subset")
    H.log(f"decode A={A} kernel={kernel}: generating")
    inp = workloads.draw_decode(cfg, device="cuda")
    rng = np.random.default_rng(52)
    inp["positions"] = rng.integers(0, C, size=A).astype(np.int32)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    H.log("  running")
    run.run(kernel=kernel)
    assert int(run.status.item()) == 0
    entries = sorted({0, 1, 65534, 65535, 65536, A - 1} | set(rng.integers(0, A, 40).tolist()))
    H.log(f"  oracle on {len(entries)} entries")
    H.full_parity(run, Kpre, Vpre, entries=entries)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))
    assert torch.isfinite(run.out.float()).all()


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
def test_prefill_66000_tokens(kernel):
    T = 66000
    cfg = workloads.config("prefill", A=1, S=2, C=T + 48, T=T, Hq=2, Hkv=1, D=64, base=1.0e4,
                           seed=53, rows_override=[1])
    H.log(f"prefill T={T} kernel={kernel}: generating")
    inp = workloads.draw_prefill(cfg, device="cuda")
    Kc, Vc = inp["Kc"], inp["Vc"]
    Kpre, Vpre = Kc.clone(), Vc.clone()
    cache = pac.Cache.wrap([Kc], [Vc])
    rows_h = np.array([1], dtype=np.int32)
    out = torch.empty_like(inp["q"])
    ws = torch.empty(pac.prefill_workspace_size(cache, 1, T, 2), dtype=torch.uint8, device="cuda")
    H.log("  running")
    pac.prefill_rope_store_attn(cache, 0, inp["q"], inp["k_new"], inp["v_new"],
                                torch.as_tensor(rows_h, device="cuda"), rows_h, out, ws,
                                cfg["base"], kernel=kernel)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    t_list = [0, 1, 127, 128, 4097, 65534, 65535, 65536, 65663, T - 1]
    H.log("  oracle on sampled query positions")
    Km = workloads.bits(Kpre[1:2]).copy()
    Vm = workloads.bits(Vpre[1:2]).copy()
    want = oracle.prefill(workloads.bits(inp["q"]), workloads.bits(inp["k_new"]),
                          workloads.bits(inp["v_new"]), [0], Km, Vm, cfg["base"], t_list=t_list)
    got = workloads.bits(out)
    H.check_output(got[0, t_list], want[0, t_list], "prefill T=66000")
    assert np.array_equal(workloads.bits(Vc[1, :T]), Vm[0, :T])
    assert ulp_dist(workloads.bits(Kc[1, :T]), Km[0, :T]).max() <= 1
    assert torch.equal(Kc[0].view(torch.int16), Kpre[0].view(torch.int16))
    assert torch.equal(Kc[1, T:].view(torch.int16), Kpre[1, T:].view(torch.int16))
    assert torch.equal(Vc[1, T:].view(torch.int16), Vpre[1, T:].view(torch.int16))


def test_decode_last_position_long_row():
    C = 131072
    cfg = workloads.config("tiny", A=2, S=3, C=C, Hq=32, Hkv=8, D=128, seed=54, base=5.0e5,
                           rows="subset")
    H.log(f"decode at position {C - 1}: generating")
    inp = workloads.draw_decode(cfg, device="cuda")
    inp["positions"] = np.array([C - 1, C - 2], dtype=np.int32)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0)
    H.log("  oracle on both entries")
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))
