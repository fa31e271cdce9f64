"""GPU parity of the equal-length batched prefill against the CPU oracle.

Bar: V store and untouched cache bytes bit-exact, rotated K store within one
BF16 ulp, BF16 output within max-abs 2e-2 and RMS 4e-3.  The matrix-core
kernel carries the FP32 rotated query as two parts in the storage type (the
high part and the rounded remainder) and rounds the softmax weights once
before its products (FP32 accumulation); the bar applies unchanged.
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


class PrefillRun:
    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        gen_dev = "cpu" if cfg["A"] * cfg["T"] * cfg["Hq"] * cfg["D"] < (1 << 24) else device
        inp = workloads.draw_prefill(cfg, device=gen_dev)
        self.q = inp["q"].to(device)
        self.k = inp["k_new"].to(device)
        self.v = inp["v_new"].to(device)
        self.Kc = inp["Kc"].to(device)
        self.Vc = inp["Vc"].to(device)
        self.rows_h = np.asarray(cfg.get("rows_override", inp["rows"]), dtype=np.int32)
        self.rows = torch.as_tensor(self.rows_h, device=device)
        self.cache = pac.Cache.wrap([self.Kc], [self.Vc])
        self.out = torch.empty_like(self.q)

    def run(self, kernel=0):
        A, T, Hq = self.q.shape[0], self.q.shape[1], self.q.shape[2]
        n = pac.prefill_workspace_size(self.cache, A, T, Hq)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.q.device)
        for r in self.rows_h:
            self.cache.reset_row(int(r))
        pac.prefill_rope_store_attn(self.cache, 0, self.q, self.k, self.v, self.rows, self.rows_h,
                                    self.out, ws, self.cfg["base"], kernel=kernel)
        torch.cuda.synchronize()
        return self.out


def parity(run, Kpre, Vpre, entries=None, t_list=None):
    """Oracle on host copies of the chosen entries (their rows' caches before the step)."""
    A, T = run.q.shape[0], run.q.shape[1]
    entries = list(range(A)) if entries is None else entries
    qb, kb, vb = workloads.bits(run.q), workloads.bits(run.k), workloads.bits(run.v)
    out = workloads.bits(run.out)
    got, want, kd = [], [], []
    for a in entries:
        r = int(run.rows_h[a])
        Km = workloads.bits(Kpre[r:r + 1]).copy()
        Vm = workloads.bits(Vpre[r:r + 1]).copy()
        o = oracle.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [0], Km, Vm, run.cfg["base"],
                           t_list=t_list, dtype=run.cfg["dtype"])
        kgot = workloads.bits(run.Kc[r, :T])
        vgot = workloads.bits(run.Vc[r, :T])
        assert np.array_equal(vgot, Vm[0, :T]), f"V store differs for entry {a}"
        d = ulp_dist(kgot, Km[0, :T])
        assert d.max() <= 1, f"K store off by {d.max()} ulp for entry {a}"
        kd.append(d.ravel())
        ts = range(T) if t_list is None else t_list
        for t in ts:
            got.append(out[a, t])
            want.append(o[0, t])
    kd = np.concatenate(kd)
    H.log(f"  K store exact fraction {np.mean(kd == 0):.6f}")
    return H.check_output(np.stack(got), np.stack(want), "prefill output",
                          dtype=run.cfg["dtype"])


def untouched(run, Kpre, Vpre):
    T = run.q.shape[1]
    Kx, Vx = Kpre.clone(), Vpre.clone()
    for r in run.rows_h:
        Kx[int(r), :T] = run.Kc[int(r), :T]
        Vx[int(r), :T] = run.Vc[int(r), :T]
    assert torch.equal(Kx.view(torch.int16), run.Kc.view(torch.int16))
    assert torch.equal(Vx.view(torch.int16), run.Vc.view(torch.int16))


SHAPES = [  # (T, Hq, Hkv, D)
    (1, 4, 2, 64), (17, 8, 2, 128), (64, 4, 4, 128), (65, 8, 2, 64), (128, 32, 8, 128),
    (129, 8, 2, 128), (200, 6, 2, 64), (333, 16, 2, 128), (97, 32, 2, 128),
]


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{t}_{q}x{k}_D{d}" for t, q, k, d in SHAPES])
def test_prefill_shapes(kernel, shape):
    T, Hq, Hkv, D = shape
    H.log(f"prefill kernel={kernel} T={T} Hq={Hq} Hkv={Hkv} D={D}")
    cfg = workloads.config("prefill", A=3, S=5, C=max(T + 7, 64), T=T, Hq=Hq, Hkv=Hkv, D=D,
                           base=1.0e4, seed=T + Hq, rows_override=[4, 0, 2])
    run = PrefillRun(cfg)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(kernel)
    assert torch.isfinite(run.out.float()).all()
    parity(run, Kpre, Vpre)
    untouched(run, Kpre, Vpre)
    for r in run.rows_h:
        assert run.cache.row_length(int(r)) == T


@pytest.mark.parametrize("A,Hkv,G", [(6, 8, 2), (5, 16, 1)], ids=["6x8_G2", "5x16_G1"])
def test_prefill_xcd_pair_chunks(A, Hkv, G):
    """Entry x kv-head pair counts that fill several chunks of pairs per XCD with a
    partial last chunk (48 pairs: 6 per XCD, chunks of 4 and 2; 80 pairs: 10 per
    XCD, chunks 4, 4, 2): every output against the oracle, every store, the rest
    of the cache untouched."""
    T, D = 150, 128
    H.log(f"prefill pair chunks A={A} Hkv={Hkv} G={G}")
    cfg = workloads.config("prefill", A=A, S=A + 2, C=T + 10, T=T, Hq=Hkv * G, Hkv=Hkv, D=D,
                           base=1.0e4, seed=A * Hkv + G, rows_override=list(range(A + 1, 0, -1))[:A])
    run = PrefillRun(cfg)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    assert torch.isfinite(run.out.float()).all()
    parity(run, Kpre, Vpre)
    untouched(run, Kpre, Vpre)


def test_prefill_full_config():
    """16 prompts x 1024 tokens, 32/8/128: every store checked, outputs of two rows
    at query positions around the tile boundaries checked against the oracle."""
    cfg = workloads.config("prefill")
    H.log("prefill full config: generating")
    run = PrefillRun(cfg)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    assert torch.isfinite(run.out.float()).all()
    H.log("prefill full config: oracle on sampled rows")
    t_list = [0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 511, 512, 767, 1000, 1022, 1023]
    parity(run, Kpre, Vpre, entries=[0, 11], t_list=t_list)
    untouched(run, Kpre, Vpre)
    # every row's stores: K within 1 ulp of the oracle, V exact (no attention computed)
    qb, kb, vb = workloads.bits(run.q), workloads.bits(run.k), workloads.bits(run.v)
    T = cfg["T"]
    for a in range(cfg["A"]):
        r = int(run.rows_h[a])
        Km = workloads.bits(Kpre[r:r + 1]).copy()
        Vm = workloads.bits(Vpre[r:r + 1]).copy()
        oracle.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [0], Km, Vm, cfg["base"], t_list=[])
        assert np.array_equal(workloads.bits(run.Vc[r, :T]), Vm[0, :T])
        assert ulp_dist(workloads.bits(run.Kc[r, :T]), Km[0, :T]).max() <= 1
    # the mfma and readable kernels agree over the whole output
    fast = workloads.bits(run.out)
    run2 = PrefillRun(cfg)
    run2.run(1)
    H.check_output(fast, workloads.bits(run2.out), "mfma vs readable (whole output)")


def test_prefill_rejects_busy_row():
    cfg = workloads.config("prefill", A=2, S=3, C=64, T=16, Hq=4, Hkv=2, D=64, base=1.0e4,
                           rows_override=[1, 2])
    run = PrefillRun(cfg)
    run.run(0)
    n = pac.prefill_workspace_size(run.cache, 2, 16, 4)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(pac.MllmError) as e:
        pac.prefill_rope_store_attn(run.cache, 0, run.q, run.k, run.v, run.rows, run.rows_h,
                                    run.out, ws, cfg["base"])
    assert e.value.name == "ROW_BUSY"
    run.cache.reset_row(1)
    run.cache.reset_row(2)
    pac.prefill_rope_store_attn(run.cache, 0, run.q, run.k, run.v, run.rows, run.rows_h,
                                run.out, ws, cfg["base"])
    torch.cuda.synchronize()


def test_decode_after_prefill():
    """Prefill T tokens, then one decode step at position T: equals the oracle's
    prefill of T + 1 tokens at its last query (within tolerance)."""
    T = 100
    cfg = workloads.config("prefill", A=2, S=2, C=128, T=T + 1, Hq=8, Hkv=2, D=128, base=5.0e5,
                           rows_override=[1, 0])
    inp = workloads.draw_prefill(cfg, device="cpu")
    dev = "cuda"
    Kc, Vc = inp["Kc"].to(dev), inp["Vc"].to(dev)
    cache = pac.Cache.wrap([Kc], [Vc])
    rows_h = np.array([1, 0], dtype=np.int32)
    rows = torch.as_tensor(rows_h, device=dev)
    q, k, v = inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev)
    out_p = torch.empty_like(q[:, :T])
    ws = torch.empty(max(256, pac.prefill_workspace_size(cache, 2, T, 8)), dtype=torch.uint8,
                     device=dev)
    pac.prefill_rope_store_attn(cache, 0, q[:, :T].contiguous(), k[:, :T].contiguous(),
                                v[:, :T].contiguous(), rows, rows_h, out_p, ws, cfg["base"])
    pos = torch.full((2,), T, dtype=torch.int32, device=dev)
    out_d = torch.empty_like(q[:, T])
    wsd = torch.empty(pac.decode_workspace_size(cache, 2, 8, T), dtype=torch.uint8, device=dev)
    pac.decode_rope_store_attn(cache, 0, q[:, T].contiguous(), k[:, T].contiguous(),
                               v[:, T].contiguous(), pos, rows, out_d, wsd, cfg["base"],
                               host_mirror=np.array([T, T, 1, 0], dtype=np.int32))
    torch.cuda.synchronize()
    assert cache.row_length(1) == T + 1 and cache.row_length(0) == T + 1
    Ko, Vo = workloads.bits(inp["Kc"]), workloads.bits(inp["Vc"])
    want = oracle.prefill(workloads.bits(inp["q"]), workloads.bits(inp["k_new"]),
                          workloads.bits(inp["v_new"]), rows_h, Ko, Vo, cfg["base"],
                          t_list=[T - 1, T])
    H.check_output(workloads.bits(out_d), want[:, T], "decode after prefill")
    H.check_output(workloads.bits(out_p[:, T - 1]), want[:, T - 1], "prefill last row")
    assert np.array_equal(workloads.bits(Vc[[1, 0], :T + 1]), Vo[[1, 0], :T + 1])
