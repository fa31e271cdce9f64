"""GPU accuracy margins at full size, measured against the CPU oracle.

1. The 16 x 1024 prefill: every row, at the tile-boundary queries and the
   first and last query of every 32-query block, under the target bar
   (max-abs 2e-2, RMS 4e-3 over the compared outputs).
2. A wide-value input family: V drawn with sigma 3 on half the kv heads and the
   queries doubled (sharper softmax), so that multi-key outputs reach
   |o| in [4, 8), where one BF16 ulp (2^-5) exceeds the 2e-2 bar.  A single
   rounding flip there fails the literal bar for any implementation whose FP32
   sums are not bit-identical to the oracle's, so the per-element bar is read as
   max(2e-2, one BF16 ulp of the oracle's value); the RMS bar is unchanged.
   Decode and prefill both run this family.
Errors are logged by |o| band.  The oracle runs entry by entry on a thread
pool (its C entry point runs without the GIL).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import positions_aware_cached_amd as pac
import workloads
from bf16util import ulp_dist, widen

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
# every tile boundary of the 64-key tiles near the start and end, plus the
# first and last query of each 32-query block of the attention kernel's work
# groups
T_LIST = sorted(set([0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 511, 512, 767, 1000, 1022, 1023] +
                    list(range(31, 1024, 32)) + list(range(32, 1024, 32))))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def _bands(got, want):
    """Max-abs and max ulp distance of the outputs by |oracle value| band (logged)."""
    g, w = widen(got, "bf16").astype(np.float64), widen(want, "bf16").astype(np.float64)
    err, ulp = np.abs(g - w), ulp_dist(got, want)
    for lo, hi in ((0, 0.5), (0.5, 1), (1, 2), (2, 4), (4, 8), (8, np.inf)):
        m = (np.abs(w) >= lo) & (np.abs(w) < hi)
        if m.any():
            H.log(f"    |o| in [{lo}, {hi}): n={int(m.sum())} max-abs {err[m].max():.3e} "
                  f"max ulp {int(ulp[m].max())} above 2e-2: {int((err[m] > 2e-2).sum())}")
    return err, w


def _check_wide(got, want, what):
    """Per element |err| <= max(2e-2, one BF16 ulp of the oracle value); RMS <= 4e-3."""
    err, w = _bands(got, want)
    mag = np.abs(w)
    one_ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 7), 0.0)
    bound = np.maximum(H.MAX_ABS, one_ulp)
    rms = float(np.sqrt(np.mean(err ** 2)))
    H.log(f"  {what}: max-abs {err.max():.3e} rms {rms:.3e}; worst err / bound "
          f"{float((err / bound).max()):.3f}")
    assert np.all(np.isfinite(widen(got, "bf16"))), what
    assert np.all(err <= bound), f"{what}: an output is beyond max(2e-2, one ulp)"
    assert rms <= H.RMS, f"{what}: rms {rms}"


def _prefill(vscale, qscale):
    cfg = workloads.config("prefill")
    A, T, Hq, Hkv = cfg["A"], cfg["T"], cfg["Hq"], cfg["Hkv"]
    inp = workloads.draw_prefill(cfg, device="cuda")
    if vscale != 1.0:
        v = inp["v_new"]
        v[:, :, :Hkv // 2] = (v[:, :, :Hkv // 2].float() * vscale).to(v.dtype)
    if qscale != 1.0:
        inp["q"] = (inp["q"].float() * qscale).to(inp["q"].dtype)
    Kp, Vp = workloads.bits(inp["Kc"]).copy(), workloads.bits(inp["Vc"]).copy()
    cache = pac.Cache.wrap([inp["Kc"]], [inp["Vc"]])
    rows_h = np.asarray(inp["rows"], dtype=np.int32)
    out = torch.empty_like(inp["q"])
    ws = torch.empty(pac.prefill_workspace_size(cache, A, T, Hq), dtype=torch.uint8,
                     device="cuda")
    pac.prefill_rope_store_attn(cache, 0, inp["q"], inp["k_new"], inp["v_new"],
                                torch.as_tensor(rows_h, device="cuda"), rows_h, out, ws,
                                cfg["base"])
    torch.cuda.synchronize()
    qb, kb, vb = (workloads.bits(inp[k]) for k in ("q", "k_new", "v_new"))
    ob = workloads.bits(out)

    def row(a):
        r = int(rows_h[a])
        Km, Vm = Kp[r:r + 1].copy(), Vp[r:r + 1].copy()
        o = oracle.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [0], Km, Vm, cfg["base"],
                           t_list=T_LIST)
        return o[0, T_LIST], ob[a, T_LIST]

    with ThreadPoolExecutor(THREADS) as pool:
        res = list(pool.map(row, range(A)))
    return np.stack([g for _, g in res]), np.stack([w for w, _ in res])


def test_prefill_every_row_full_config():
    """All 16 rows of the 16 x 1024 prefill at 22 query positions each."""
    H.log("prefill 16 x 1024, every row vs the oracle")
    got, want = _prefill(1.0, 1.0)
    _bands(got, want)
    H.check_output(got, want, "prefill, every row")


def test_prefill_wide_values():
    H.log("prefill 16 x 1024, V x3 on half the kv heads, Q x2")
    got, want = _prefill(3.0, 2.0)
    _check_wide(got, want, "prefill wide values")


def test_decode_wide_values():
    H.log("decode Llama-like batch, V x3 on half the kv heads, Q x2")
    cfg = workloads.config("llama3_8b")
    Hkv, D = cfg["Hkv"], cfg["D"]
    inp = workloads.draw_decode(cfg, device="cuda")
    for k in ("Vc", "v_new"):
        x = inp[k]
        x[..., :Hkv // 2, :] = (x[..., :Hkv // 2, :].float() * 3.0).to(x.dtype)
    inp["q"] = (inp["q"].float() * 2.0).to(inp["q"].dtype)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0)
    qb, kb, vb = (workloads.bits(t) for t in (run.q, run.k_new, run.v_new))
    ob = workloads.bits(run.out)

    def entry(a):
        p, r = int(run.pos_h[a]), int(run.rows_h[a])
        Km = workloads.bits(Kpre[r, :p + 1]).reshape(1, p + 1, Hkv, D).copy()
        Vm = workloads.bits(Vpre[r, :p + 1]).reshape(1, p + 1, Hkv, D).copy()
        return oracle.decode_step(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [p], [0], Km, Vm,
                                  cfg["base"])[0], ob[a]

    with ThreadPoolExecutor(THREADS) as pool:
        res = list(pool.map(entry, range(cfg["A"])))
    _check_wide(np.stack([g for _, g in res]), np.stack([w for w, _ in res]),
                "decode wide values")
