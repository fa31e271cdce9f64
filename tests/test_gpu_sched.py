"""The slot manager driving the batched kernels, cross-checked against serial
B=1 execution of every request (the pages' divergent-position oracle runs each
row as its own B=1 view: microLLM-rocm ARCHITECTURE.md, "Tensor ownership
boundary").

A trace of requests with different prompt lengths, output lengths, a stop and
cancellations (queued and active) runs through mllm_sched_*: at each boundary
the admitted requests are prefilled in equal-length groups and the decode list
runs as one batched decode call on the shared cache.  Each request is also run
alone in a private one-row cache with the same inputs.  Checked: every output
of every request, batched vs alone, to the output bar; each request's stored
K/V rows, bit for bit, when it leaves its row; outputs of sampled requests
against the CPU oracle; and the end state (all rows free and reset).
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import positions_aware_cached_amd as pac
import workloads

pytestmark = pytest.mark.gpu

S, CAP, HQ, HKV, D, BASE = 4, 96, 8, 2, 128, 1.0e4
# (request id, prompt length, new tokens)
REQUESTS = [(0, 9, 6), (1, 5, 0), (2, 9, 3), (3, 17, 10), (4, 33, 4), (5, 5, 8), (6, 40, 2),
            (7, 12, 12), (8, 9, 5), (9, 20, 7)]
STOP_AFTER = {3: 4}          # request 3 is stopped after 4 decode steps
CANCEL_AFTER = {7: 2}        # request 7 is cancelled after 2 decode steps
CANCEL_QUEUED_AT = {6: 1}    # request 6 is cancelled while queued, before boundary 1


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def _tokens(rid, n, dtype):
    g = torch.Generator().manual_seed(7000 + rid)
    t = lambda h: torch.randn((n, h, D), generator=g).to(workloads.TORCH_DTYPES[dtype])
    return t(HQ).cuda(), t(HKV).cuda(), t(HKV).cuda()


def _cache(rows, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    t = lambda: torch.randn((rows, CAP, HKV, D), generator=g).to(
        workloads.TORCH_DTYPES[dtype]).cuda()
    K, V = t(), t()
    return pac.Cache.wrap([K], [V]), K, V


def _ws_decode(cache, A):
    return torch.empty(max(256, pac.decode_workspace_size(cache, A, HQ, CAP - 1)),
                       dtype=torch.uint8, device="cuda")


def _prefill(cache, q, k, v, rows):
    A, T = q.shape[0], q.shape[1]
    out = torch.empty_like(q)
    ws = torch.empty(max(256, pac.prefill_workspace_size(cache, A, T, HQ)), dtype=torch.uint8,
                     device="cuda")
    rows_h = np.asarray(rows, dtype=np.int32)
    pac.prefill_rope_store_attn(cache, 0, q.contiguous(), k.contiguous(), v.contiguous(),
                                torch.as_tensor(rows_h, device="cuda"), rows_h, out, ws, BASE)
    return out


def _decode(cache, q, k, v, pos, rows):
    A = q.shape[0]
    out = torch.empty_like(q)
    pos_h, rows_h = np.asarray(pos, np.int32), np.asarray(rows, np.int32)
    pac.decode_rope_store_attn(cache, 0, q.contiguous(), k.contiguous(), v.contiguous(),
                               torch.as_tensor(pos_h, device="cuda"),
                               torch.as_tensor(rows_h, device="cuda"), out, _ws_decode(cache, A),
                               BASE, host_mirror=np.concatenate([pos_h, rows_h]))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_scheduled_batch_equals_serial_b1(dtype):
    H.log(f"scheduler trace, {dtype}")
    toks = {rid: _tokens(rid, p + n, dtype) for rid, p, n in REQUESTS}
    spec = {rid: (p, n) for rid, p, n in REQUESTS}
    cache, Kc, Vc = _cache(S, dtype, 1)
    sched = pac.Scheduler(cache, 64)
    for rid, p, n in REQUESTS:
        sched.submit(rid, p, n)
    batched = {rid: {} for rid in spec}   # rid -> {position: output [Hq, D] bits}
    retired_rows = {}                     # rid -> (K, V) rows [len, Hkv, D] at retirement
    reasons, decoded = {}, {rid: 0 for rid in spec}
    step = 0
    while True:
        for rid, at in CANCEL_QUEUED_AT.items():
            if at == step:
                sched.cancel(rid)
                reasons[rid] = "cancelled while queued"
        admitted, decode, retired = sched.boundary()
        for rid, row, why in retired:
            n = cache.row_length(row)     # already reset: use the positions it held
            held = spec[rid][0] + decoded[rid]
            assert n == 0
            retired_rows[rid] = (Kc[row, :held].clone(), Vc[row, :held].clone())
            reasons[rid] = pac.END_REASONS[why]
        if not (admitted or decode) and sched.counts() == (0, 0):
            break
        # equal-length prefill groups
        groups = {}
        for rid, row, p in admitted:
            groups.setdefault(p, []).append((rid, row))
        for p, members in groups.items():
            q = torch.stack([toks[rid][0][:p] for rid, _ in members])
            k = torch.stack([toks[rid][1][:p] for rid, _ in members])
            v = torch.stack([toks[rid][2][:p] for rid, _ in members])
            out = _prefill(cache, q, k, v, [row for _, row in members])
            for a, (rid, _) in enumerate(members):
                for t in range(p):
                    batched[rid][t] = workloads.bits(out[a, t])
        if decode:
            q = torch.stack([toks[rid][0][pos] for rid, _, pos in decode])
            k = torch.stack([toks[rid][1][pos] for rid, _, pos in decode])
            v = torch.stack([toks[rid][2][pos] for rid, _, pos in decode])
            out = _decode(cache, q, k, v, [pos for _, _, pos in decode],
                          [row for _, row, _ in decode])
            for a, (rid, row, pos) in enumerate(decode):
                assert pos == spec[rid][0] + decoded[rid]
                batched[rid][pos] = workloads.bits(out[a])
                decoded[rid] += 1
                if STOP_AFTER.get(rid) == decoded[rid]:
                    sched.stop(rid)
                if CANCEL_AFTER.get(rid) == decoded[rid]:
                    sched.cancel(rid)
        step += 1
        assert step < 200
    torch.cuda.synchronize()
    H.log(f"  {step} steps; ends: {reasons}")
    assert reasons[1] == "length" and reasons[0] == "length" and reasons[3] == "stop"
    assert reasons[6] == "cancelled while queued" and reasons[7] == "cancel"
    assert decoded[3] == 4 and decoded[6] == 0 and decoded[0] == 6 and decoded[7] == 2
    assert all(cache.row_length(r) == 0 for r in range(S))

    # every request alone in a one-row cache, same inputs, same kernels
    got, want = [], []
    for rid, (p, _) in spec.items():
        if rid == 6:
            continue
        solo, Ks, Vs = _cache(1, dtype, 2)
        q, k, v = (x[:p][None] for x in toks[rid])
        o = _prefill(solo, q, k, v, [0])
        for t in range(p):
            got.append(batched[rid][t])
            want.append(workloads.bits(o[0, t]))
        for i in range(decoded[rid]):
            pos = p + i
            q, k, v = (x[pos][None] for x in toks[rid])
            o = _decode(solo, q, k, v, [pos], [0])
            got.append(batched[rid][pos])
            want.append(workloads.bits(o[0]))
        held = p + decoded[rid]
        Kb, Vb = retired_rows[rid]
        assert torch.equal(Kb.view(torch.int16), Ks[0, :held].view(torch.int16)), rid
        assert torch.equal(Vb.view(torch.int16), Vs[0, :held].view(torch.int16)), rid
    H.check_output(np.stack(got), np.stack(want), "batched vs serial B=1", dtype=dtype)

    # the CPU oracle on two requests, serially (B = 1 rows, as the pages' oracle)
    for rid in (3, 9):
        p, _ = spec[rid]
        n = p + decoded[rid]
        qb, kb, vb = (workloads.bits(x[:n]) for x in toks[rid])
        K0 = np.zeros((1, CAP, HKV, D), dtype=np.uint16)
        V0 = np.zeros((1, CAP, HKV, D), dtype=np.uint16)
        o = oracle.prefill(qb[None], kb[None], vb[None], [0], K0, V0, BASE, dtype=dtype)
        H.check_output(np.stack([batched[rid][t] for t in range(n)]), o[0],
                       f"request {rid} vs oracle", dtype=dtype)
