"""GPU parity of the decode step against the CPU oracle (through the C ABI).

Bar: V store and every untouched cache byte bit-exact, rotated K store within
one BF16 ulp, BF16 output within max-abs 2e-2 and RMS 4e-3 over the whole
output.  Full-size configurations are checked entry by entry (the oracle runs
on a host copy of each row's prefix taken before the step).
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


def small_case(D, Hq, Hkv, positions, C, S=None, seed=0, inactive="normal"):
    A = len(positions)
    S = S or A + 3
    cfg = workloads.config("tiny", A=A, S=S, C=C, Hq=Hq, Hkv=Hkv, D=D, seed=seed,
                           inactive=inactive)
    inp = workloads.draw_decode(cfg, device="cpu")
    inp["positions"] = np.asarray(positions, dtype=np.int32)
    return cfg, inp


@pytest.mark.parametrize("kernel", [0, 1], ids=["tuned", "readable"])
@pytest.mark.parametrize("mirror", [True, False], ids=["mirror", "nomirror"])
def test_tiny_parity(kernel, mirror):
    cfg = workloads.config("tiny")
    H.log(f"tiny kernel={kernel} mirror={mirror}")
    inp = workloads.draw_decode(cfg, device="cpu")
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
@pytest.mark.parametrize("waves", [1, 5, 64, 0], ids=["w1", "w5", "w64", "wdev"])
def test_edge_positions(D, heads, waves):
    """Every tile boundary, with one wave walking all segments, waves splitting
    segments mid-way, and the device default (more waves than tiles)."""
    Hq, Hkv = heads
    H.log(f"edge D={D} Hq={Hq} Hkv={Hkv} waves={waves}")
    cfg, inp = small_case(D, Hq, Hkv, EDGE_POS, C=640, seed=D + Hq + waves)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0, waves=waves)
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


@pytest.mark.parametrize("case", ["start_only_ranges", "weighted_short_rows"])
def test_short_rows_unit_plan(case):
    """Short rows on the device default launch, where the plan counts each
    segment start as a unit of work: about one unit and a half per group, so
    some groups own only a segment start and no tile; and short rows with
    enough tiles for the two-per-unit weighted split."""
    rng = np.random.default_rng(11 if case == "start_only_ranges" else 12)
    if case == "start_only_ranges":
        positions = rng.integers(0, 96, 100)     # 1..3 tiles per row
    else:
        positions = rng.integers(0, 640, 200)    # 1..20 tiles per row
    H.log(f"unit plan {case}: A={len(positions)}")
    cfg, inp = small_case(128, 32, 8, positions, C=640, seed=len(positions))
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=0, waves=0)
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))


@pytest.mark.parametrize("D", [64, 128])
def test_readable_edges(D):
    H.log(f"readable edge D={D}")
    cfg, inp = small_case(D, 8, 2, EDGE_POS, C=640, seed=3)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(kernel=1)
    H.full_parity(run, Kpre, Vpre)


def test_sentinel_never_read():
    """NaN sentinels in inactive rows and beyond every prefix never reach the output."""
    H.log("sentinel")
    cfg, inp = small_case(128, 32, 8, [5, 300, 0, 1023, 64], C=1024, S=9, seed=11)
    base_run = H.DecodeRun(inp, cfg)
    base_run.run()
    ref = base_run.out.clone()
    Kc, Vc = inp["Kc"].clone(), inp["Vc"].clone()
    nan = torch.tensor(workloads.NAN_SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    keep = torch.zeros(Kc.shape[:2], dtype=torch.bool)
    for p, r in zip(inp["positions"], inp["rows"]):
        keep[r, :p] = True
    Kc[~keep] = nan
    Vc[~keep] = nan
    inp2 = dict(inp, Kc=Kc, Vc=Vc)
    for kernel in (0, 1):
        run = H.DecodeRun(inp2, cfg)
        run.run(kernel=kernel)
        assert torch.isfinite(run.out.float()).all()
        if kernel == 0:
            assert torch.equal(run.out.view(torch.int16), ref.view(torch.int16))


def test_idempotent_deterministic_wave_invariant():
    H.log("idempotence / determinism / wave-count invariance")
    cfg, inp = small_case(128, 32, 8, [100, 2047, 900, 4095, 1], C=4096, S=6, seed=21)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    o1 = run.run().clone()
    K1, V1 = run.Kc.clone(), run.Vc.clone()
    o2 = run.run().clone()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(K1.view(torch.int16), run.Kc.view(torch.int16))
    assert torch.equal(V1.view(torch.int16), run.Vc.view(torch.int16))
    outs = []
    for waves in (1, 3, 100, 4096):
        outs.append(H.workloads.bits(run.run(waves=waves)))
    for o in outs[1:]:
        H.check_output(o, outs[0], "wave-count invariance")
    H.full_parity(run, Kpre, Vpre)


def test_device_index_error_without_mirror():
    """Without a host mirror an out-of-range entry is skipped, its output is NaN,
    the status word is set, and the other entries are unaffected."""
    H.log("device-side index error")
    cfg, inp = small_case(64, 4, 2, [3, 10, 20, 7], C=64, S=6, seed=5)
    inp["positions"] = np.array([3, 64, 20, 7], dtype=np.int32)   # entry 1 out of range
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    run.run(mirror=False)
    assert int(run.status.item()) == 1
    assert torch.isnan(run.out[1].float()).all()
    assert torch.isfinite(run.out[[0, 2, 3]].float()).all()
    good = [0, 2, 3]
    want = H.oracle_rows(run.q, run.k_new, run.v_new, Kpre, Vpre, run.pos_h, run.rows_h,
                         cfg["base"], good)
    got = workloads.bits(run.out)
    H.check_output(got[good], np.stack([want[a][0] for a in good]), "valid entries")
    H.check_untouched(run, Kpre, Vpre, [(run.rows_h[a], run.pos_h[a]) for a in good])


def test_row_lengths_and_engine_owned_cache():
    """Host mirror updates row lengths; an engine-owned cache gives the same result."""
    import positions_aware_cached_amd as pac
    H.log("engine-owned cache")
    cfg, inp = small_case(128, 8, 2, [7, 100, 33], C=128, S=4, seed=8)
    run = H.DecodeRun(inp, cfg)
    run.run()
    for p, r in zip(run.pos_h, run.rows_h):
        assert run.cache.row_length(int(r)) == p + 1
    run.cache.reset_row(int(run.rows_h[0]))
    assert run.cache.row_length(int(run.rows_h[0])) == 0
    owned = pac.Cache.alloc(1, 4, 128, 2, 128, device=0)
    kp, vp = owned.layer_ptrs(0)
    nbytes = 4 * 128 * 2 * 128 * 2
    for ptr, src in ((kp, inp["Kc"]), (vp, inp["Vc"])):
        H.copy_to_device_ptr(ptr, src, nbytes)
    o = torch.empty_like(run.out)
    ws = torch.empty(pac.decode_workspace_size(owned, 3, 8, -1), dtype=torch.uint8,
                     device="cuda")
    pac.decode_rope_store_attn(owned, 0, run.q, run.k_new, run.v_new, run.pos, run.rows, o, ws,
                               cfg["base"])
    torch.cuda.synchronize()
    ref = H.DecodeRun(inp, cfg)
    ref.run(mirror=False)
    assert torch.equal(o.view(torch.int16), ref.out.view(torch.int16))
    owned.free()


@pytest.mark.parametrize("name", ["llama3_8b", "ragged", "long"])
def test_full_config_parity(name):
    cfg = workloads.config(name)
    H.log(f"full config {name}: generating on device")
    inp = workloads.draw_decode(cfg, device="cuda")
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    H.log(f"full config {name}: running")
    run.run()
    H.log(f"full config {name}: oracle on every entry")
    H.full_parity(run, Kpre, Vpre)
    H.check_untouched(run, Kpre, Vpre, list(zip(run.rows_h, run.pos_h)))
    if name == "ragged":
        # inactive rows hold the sentinel and stayed bit-identical (checked above);
        # outputs must be finite, so no sentinel was read
        assert torch.isfinite(run.out.float()).all()


@pytest.mark.parametrize("kernel", [0, 1], ids=["tuned", "readable"])
def test_graph_capture_replay(kernel):
    """The step captured into a HIP graph (it allocates nothing, memsets nothing
    and plans on the device) replays to the eager result, bit for bit, on
    every replay, with eager work and synchronizations in between."""
    import positions_aware_cached_amd as pac
    H.log(f"graph capture kernel={kernel}")
    cfg, inp = small_case(128, 32, 8, [100, 2047, 900, 4095, 1, 333], C=4096, S=8, seed=31)
    run = H.DecodeRun(inp, cfg)
    Kpre, Vpre = run.snapshot()
    want = run.run(kernel=kernel).clone()
    Kw, Vw = run.Kc.clone(), run.Vc.clone()
    H.full_parity(run, Kpre, Vpre)
    A, Hq, _ = run.q.shape
    ws = torch.empty(pac.decode_workspace_size(run.cache, A, Hq, -1, 0, kernel), dtype=torch.uint8,
                     device="cuda")
    mirror = np.concatenate([run.pos_h, run.rows_h])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        pac.decode_rope_store_attn(run.cache, 0, run.q, run.k_new, run.v_new, run.pos, run.rows,
                                   run.out, ws, cfg["base"], host_mirror=mirror, kernel=kernel)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pac.decode_rope_store_attn(run.cache, 0, run.q, run.k_new, run.v_new, run.pos, run.rows,
                                   run.out, ws, cfg["base"], host_mirror=mirror, kernel=kernel)
    for rep in range(3):
        run.out.zero_()
        run.Kc.copy_(Kpre)
        run.Vc.copy_(Vpre)
        ws.fill_(0xA5)  # the workspace carries nothing from one call to the next
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
        assert torch.equal(run.Kc.view(torch.int16), Kw.view(torch.int16)), f"replay {rep} K"
        assert torch.equal(run.Vc.view(torch.int16), Vw.view(torch.int16)), f"replay {rep} V"
