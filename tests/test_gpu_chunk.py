"""GPU parity of the prefill chunk (per-entry start positions and lengths)
against the CPU oracle.

Bar: V store and untouched cache bytes bit-exact, rotated K store within one
BF16 ulp, BF16 output within max-abs 2e-2 and RMS 4e-3; output rows past an
entry's length keep their prior bits.  The cached prefix before each start is
random BF16 data drawn by the seeded generators.
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

SENT = np.uint16(workloads.NAN_SENTINEL)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


class ChunkRun:
    def __init__(self, cfg, starts, lens, rows, device="cuda"):
        self.cfg = cfg
        gen_dev = "cpu" if cfg["A"] * cfg["T"] * cfg["Hq"] * cfg["D"] < (1 << 24) else device
        inp = workloads.draw_prefill(cfg, device=gen_dev)
        self.q = inp["q"].to(device)
        self.k = inp["k_new"].to(device)
        self.v = inp["v_new"].to(device)
        self.Kc = inp["Kc"].to(device)
        self.Vc = inp["Vc"].to(device)
        self.starts = np.asarray(starts, dtype=np.int32)
        self.lens = np.asarray(lens, dtype=np.int32)
        self.rows_h = np.asarray(rows, dtype=np.int32)
        self.meta_h = np.concatenate([self.starts, self.lens, self.rows_h]).astype(np.int32)
        self.meta = torch.as_tensor(self.meta_h, device=device)
        self.cache = pac.Cache.wrap([self.Kc], [self.Vc])
        # raw bits: a NaN filled through a float value would be canonicalised
        self.out = torch.full(self.q.shape, int(SENT), dtype=torch.int16,
                              device=device).view(self.q.dtype)

    def run(self, kernel=0):
        A, T, Hq = self.q.shape[0], self.q.shape[1], self.q.shape[2]
        n = pac.prefill_workspace_size(self.cache, A, T, Hq)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.q.device)
        pac.prefill_chunk_rope_store_attn(self.cache, 0, self.q, self.k, self.v, self.meta,
                                          self.meta_h, self.out, ws, self.cfg["base"],
                                          kernel=kernel)
        torch.cuda.synchronize()
        return self.out


def parity(run, Kpre, Vpre, entries=None, t_list=None):
    """Oracle per entry on host copies of its row before the call; checks the
    stores of every token of the chosen entries and the outputs of t_list (all
    tokens when None) within the entry's length."""
    A = run.q.shape[0]
    entries = list(range(A)) if entries is None else entries
    qb, kb, vb = workloads.bits(run.q), workloads.bits(run.k), workloads.bits(run.v)
    out = workloads.bits(run.out)
    got, want, kd = [], [], []
    for a in entries:
        r, s, n = int(run.rows_h[a]), int(run.starts[a]), int(run.lens[a])
        Km = workloads.bits(Kpre[r:r + 1]).copy()
        Vm = workloads.bits(Vpre[r:r + 1]).copy()
        ts = list(range(n)) if t_list is None else [t for t in t_list if t < n]
        o = oracle.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [0], Km, Vm, run.cfg["base"],
                           t_list=ts, starts=[s], lens=[n], dtype=run.cfg["dtype"])
        vgot = workloads.bits(run.Vc[r, s:s + n])
        assert np.array_equal(vgot, Vm[0, s:s + n]), f"V store differs for entry {a}"
        d = ulp_dist(workloads.bits(run.Kc[r, s:s + n]), Km[0, s:s + n])
        assert d.max() <= 1, f"K store off by {d.max()} ulp for entry {a}"
        kd.append(d.ravel())
        assert (out[a, n:] == SENT).all(), f"entry {a}: output rows past its length written"
        for t in ts:
            got.append(out[a, t])
            want.append(o[0, t])
    H.log(f"  K store exact fraction {np.mean(np.concatenate(kd) == 0):.6f}")
    return H.check_output(np.stack(got), np.stack(want), "chunk output", dtype=run.cfg["dtype"])


def untouched(run, Kpre, Vpre):
    Kx, Vx = Kpre.clone(), Vpre.clone()
    for a in range(run.q.shape[0]):
        r, s, n = int(run.rows_h[a]), int(run.starts[a]), int(run.lens[a])
        Kx[r, s:s + n] = run.Kc[r, s:s + n]
        Vx[r, s:s + n] = run.Vc[r, s:s + n]
    assert torch.equal(Kx.view(torch.int16), run.Kc.view(torch.int16))
    assert torch.equal(Vx.view(torch.int16), run.Vc.view(torch.int16))


# (T, Hq, Hkv, D, starts, lengths): starts on and beside 32/64-key tile edges,
# a start at 0 (fresh prompt) beside nonzero ones, lengths of one token, of
# the whole chunk and ragged between; rows [5, 0, 3, 1] of a 6-slot cache.
CASES = [
    (1, 4, 2, 64, [0, 5, 63, 64], [1, 1, 1, 1]),
    (17, 8, 2, 128, [0, 1, 31, 100], [17, 16, 1, 17]),
    (64, 4, 4, 128, [63, 64, 65, 0], [64, 33, 64, 64]),
    (65, 8, 2, 64, [127, 2, 500, 129], [65, 64, 1, 65]),
    (128, 32, 8, 128, [128, 7, 0, 300], [128, 127, 128, 100]),
    (200, 6, 2, 64, [55, 0, 256, 511], [200, 129, 72, 200]),
    (333, 16, 2, 128, [1000, 333, 17, 0], [333, 250, 333, 128]),
]


def _case_cfg(T, Hq, Hkv, D, starts, lens, seed):
    C = max(s + n for s, n in zip(starts, lens)) + 7
    return workloads.config("prefill", A=4, S=6, C=C, T=T, Hq=Hq, Hkv=Hkv, D=D, base=1.0e4,
                            seed=seed)


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_{c[1]}x{c[2]}_D{c[3]}" for c in CASES])
def test_chunk_cases(kernel, case):
    T, Hq, Hkv, D, starts, lens = case
    H.log(f"chunk kernel={kernel} T={T} Hq={Hq} Hkv={Hkv} D={D} starts={starts} lens={lens}")
    cfg = _case_cfg(T, Hq, Hkv, D, starts, lens, seed=T + 3 * Hq)
    rows = [5, 0, 3, 1]
    run = ChunkRun(cfg, starts, lens, rows)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    for r in rows:
        run.cache.reset_row(r)
    run.run(kernel)
    parity(run, Kpre, Vpre)
    untouched(run, Kpre, Vpre)
    for a, r in enumerate(rows):
        assert run.cache.row_length(r) == starts[a] + lens[a]


def test_chunk_at_zero_is_prefill():
    """Starts 0 and full lengths on empty rows: the same bits as the prefill call."""
    cfg = workloads.config("prefill", A=3, S=4, C=300, T=257, Hq=8, Hkv=2, D=128, base=5.0e5,
                           seed=21)
    rows = [2, 0, 3]
    run = ChunkRun(cfg, [0, 0, 0], [257] * 3, rows)
    K0, V0 = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    Kc, Vc = K0.clone(), V0.clone()
    cache = pac.Cache.wrap([Kc], [Vc])
    out = torch.empty_like(run.q)
    ws = torch.empty(pac.prefill_workspace_size(cache, 3, 257, 8), dtype=torch.uint8,
                     device="cuda")
    rows_d = torch.as_tensor(np.array(rows, dtype=np.int32), device="cuda")
    pac.prefill_rope_store_attn(cache, 0, run.q, run.k, run.v, rows_d, np.array(rows, np.int32),
                                out, ws, cfg["base"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), run.out.view(torch.int16))
    assert torch.equal(Kc.view(torch.int16), run.Kc.view(torch.int16))
    assert torch.equal(Vc.view(torch.int16), run.Vc.view(torch.int16))


def test_chunks_in_sequence():
    """A prompt prefilled in three chunks of different sizes, then one decode
    step: every output within the bar of the oracle's single pass over the whole
    sequence (the oracle never sees a value the GPU produced)."""
    T1, T2, T3 = 100, 37, 64
    Ttot = T1 + T2 + T3
    cfg = workloads.config("prefill", A=2, S=3, C=256, T=Ttot + 1, Hq=8, Hkv=2, D=128,
                           base=5.0e5, seed=22)
    inp = workloads.draw_prefill(cfg, device="cpu")
    dev = "cuda"
    Kc, Vc = inp["Kc"].to(dev), inp["Vc"].to(dev)
    cache = pac.Cache.wrap([Kc], [Vc])
    rows = np.array([2, 0], dtype=np.int32)
    q, k, v = inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev)
    outs = []
    s = 0
    for n in (T1, T2, T3):
        meta_h = np.array([s, s, n, n, rows[0], rows[1]], dtype=np.int32)
        o = torch.empty_like(q[:, s:s + n])
        ws = torch.empty(pac.prefill_workspace_size(cache, 2, n, 8), dtype=torch.uint8,
                         device=dev)
        pac.prefill_chunk_rope_store_attn(cache, 0, q[:, s:s + n], k[:, s:s + n], v[:, s:s + n],
                                          torch.as_tensor(meta_h, device=dev), meta_h, o, ws,
                                          cfg["base"])
        outs.append(o)
        s += n
    pos = torch.full((2,), Ttot, dtype=torch.int32, device=dev)
    out_d = torch.empty_like(q[:, Ttot])
    wsd = torch.empty(pac.decode_workspace_size(cache, 2, 8, Ttot), dtype=torch.uint8,
                      device=dev)
    pac.decode_rope_store_attn(cache, 0, q[:, Ttot].contiguous(), k[:, Ttot].contiguous(),
                               v[:, Ttot].contiguous(), pos, torch.as_tensor(rows, device=dev),
                               out_d, wsd, cfg["base"],
                               host_mirror=np.array([Ttot, Ttot, rows[0], rows[1]], np.int32))
    torch.cuda.synchronize()
    assert cache.row_length(2) == Ttot + 1 and cache.row_length(0) == Ttot + 1
    Ko, Vo = workloads.bits(inp["Kc"]), workloads.bits(inp["Vc"])
    want = oracle.prefill(workloads.bits(inp["q"]), workloads.bits(inp["k_new"]),
                          workloads.bits(inp["v_new"]), rows, Ko, Vo, cfg["base"])
    got = workloads.bits(torch.cat(outs, dim=1))
    H.check_output(got, want[:, :Ttot], "three chunks")
    H.check_output(workloads.bits(out_d), want[:, Ttot], "decode after chunks")
    for r in rows:
        assert np.array_equal(workloads.bits(Vc[r, :Ttot + 1]), Vo[r, :Ttot + 1])
        assert ulp_dist(workloads.bits(Kc[r, :Ttot + 1]), Ko[r, :Ttot + 1]).max() <= 1


@pytest.mark.parametrize("A,Hq,Hkv", [(256, 8, 2), (260, 8, 2), (257, 6, 2)],
                         ids=["256_G4", "260_G4", "257_G3"])
def test_chunk_many_entries(A, Hq, Hkv):
    """More entries than the attention kernel's schedule takes heaviest first
    (256): 256 entries still reordered, 257 and 260 in index order; four query
    heads per work group (G = 4) and one (G = 3).  Every output and store of
    every entry against the oracle."""
    rng = np.random.default_rng(7000 + A + Hq)
    T = 16
    lens = rng.integers(1, T + 1, A).astype(np.int32)
    lens[:3] = [1, T, T]
    starts = rng.integers(0, 200, A).astype(np.int32)
    starts[:3] = [0, 0, 190]
    rows = rng.permutation(A + 2)[:A].astype(np.int32)
    C = int((starts + lens).max()) + 5
    cfg = workloads.config("prefill", A=A, S=A + 2, C=C, T=T, Hq=Hq, Hkv=Hkv, D=64,
                           base=1.0e4, seed=7100 + A)
    H.log(f"chunk many entries A={A} Hq={Hq} Hkv={Hkv}")
    run = ChunkRun(cfg, starts, lens, rows)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    parity(run, Kpre, Vpre)
    untouched(run, Kpre, Vpre)


def test_chunk_full_config():
    """16 rows, chunks of 128..512 tokens at starts in [0, 3072], 32/8/128: every
    store checked, outputs of three entries at sampled queries checked against
    the oracle, and the two kernels agree over every written output."""
    cfg = workloads.config("chunk")
    starts, lens, rows = workloads.draw_chunk_meta(cfg)
    H.log(f"chunk full config: starts={starts.tolist()} lens={lens.tolist()}")
    run = ChunkRun(cfg, starts, lens, rows)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    run.run(0)
    H.log("chunk full config: oracle on sampled entries")
    t_list = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 200, 255, 256, 300, 383, 384, 437, 511]
    longest = int(np.argmax(lens))
    latest = int(np.argmax(starts + lens))
    shortest = int(np.argmin(lens))
    parity(run, Kpre, Vpre, entries=sorted({longest, latest, shortest}), t_list=t_list)
    untouched(run, Kpre, Vpre)
    qb, kb, vb = workloads.bits(run.q), workloads.bits(run.k), workloads.bits(run.v)
    for a in range(cfg["A"]):
        r, s, n = int(rows[a]), int(starts[a]), int(lens[a])
        Km = workloads.bits(Kpre[r:r + 1]).copy()
        Vm = workloads.bits(Vpre[r:r + 1]).copy()
        oracle.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [0], Km, Vm, cfg["base"],
                       t_list=[], starts=[s], lens=[n])
        assert np.array_equal(workloads.bits(run.Vc[r, s:s + n]), Vm[0, s:s + n])
        assert ulp_dist(workloads.bits(run.Kc[r, s:s + n]), Km[0, s:s + n]).max() <= 1
    fast = workloads.bits(run.out)
    run2 = ChunkRun(cfg, starts, lens, rows)
    run2.run(1)
    slow = workloads.bits(run2.out)
    got = np.concatenate([fast[a, :lens[a]] for a in range(cfg["A"])])
    ref = np.concatenate([slow[a, :lens[a]] for a in range(cfg["A"])])
    H.check_output(got, ref, "mfma vs readable (every written output)")
    assert (fast == slow)[np.arange(fast.shape[1])[None, :] >= lens[:, None]].all()


@pytest.mark.parametrize("kernel", [0, 1], ids=["mfma", "readable"])
def test_chunk_graph_capture_replay(kernel):
    """A prefill chunk captured into a HIP graph (the call allocates and memsets
    nothing) replays to the eager result, stores and output bit for bit, on
    every replay, with eager work and synchronizations in between."""
    T, Hq, Hkv, D = 96, 8, 2, 128
    starts, lens, rows = [0, 40, 130, 7], [96, 57, 1, 80], [5, 0, 3, 1]
    H.log(f"chunk graph capture kernel={kernel}")
    cfg = _case_cfg(T, Hq, Hkv, D, starts, lens, seed=41)
    run = ChunkRun(cfg, starts, lens, rows)
    Kpre, Vpre = run.Kc.clone(), run.Vc.clone()
    want = run.run(kernel).clone()
    Kw, Vw = run.Kc.clone(), run.Vc.clone()
    parity(run, Kpre, Vpre)
    A = run.q.shape[0]
    ws = torch.empty(max(256, pac.prefill_workspace_size(run.cache, A, T, Hq)), dtype=torch.uint8,
                     device="cuda")

    def call():
        pac.prefill_chunk_rope_store_attn(run.cache, 0, run.q, run.k, run.v, run.meta,
                                          run.meta_h, run.out, ws, cfg["base"], kernel=kernel)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        run.out.view(torch.int16).fill_(int(SENT))
        run.Kc.copy_(Kpre)
        run.Vc.copy_(Vpre)
        ws.fill_(0x5A)  # the workspace carries nothing from one call to the next
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
        assert torch.equal(run.Kc.view(torch.int16), Kw.view(torch.int16)), f"replay {rep} K"
        assert torch.equal(run.Vc.view(torch.int16), Vw.view(torch.int16)), f"replay {rep} V"
