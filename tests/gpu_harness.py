"""Shared helpers of the GPU parity tests (imported by tests/test_gpu_*.py).

Inputs come from the seeded generators in `workloads`; expected values come
only from the CPU oracle (`oracle`) run on host copies of those inputs.  The
HIP path is reached only through the C ABI binding.
"""
import numpy as np
import torch

import oracle
import positions_aware_cached_amd as pac
import workloads
from bf16util import ulp_dist, widen

# Acceptance bar for the attention output (whole output tensor), BF16 or FP16.
MAX_ABS = 2e-2
RMS = 4e-3


def log(msg):
    print(msg, flush=True)


class DecodeRun:
    """Device state of one decode step: inputs, cache, workspace, outputs."""

    def __init__(self, inp, cfg, device="cuda"):
        self.cfg = cfg
        self.inp = inp
        dev = torch.device(device)
        self.q = inp["q"].to(dev)
        self.k_new = inp["k_new"].to(dev)
        self.v_new = inp["v_new"].to(dev)
        self.Kc = inp["Kc"].to(dev)
        self.Vc = inp["Vc"].to(dev)
        self.pos_h = np.asarray(inp["positions"], dtype=np.int32)
        self.rows_h = np.asarray(inp["rows"], dtype=np.int32)
        self.pos = torch.as_tensor(self.pos_h, device=dev)
        self.rows = torch.as_tensor(self.rows_h, device=dev)
        self.cache = pac.Cache.wrap([self.Kc], [self.Vc])
        A, Hq, D = self.q.shape
        self.out = torch.empty((A, Hq, D), dtype=self.q.dtype, device=dev)
        self.dtype = cfg.get("dtype", "bf16")
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)

    def snapshot(self):
        return self.Kc.clone(), self.Vc.clone()

    def run(self, kernel=0, waves=0, mirror=True, max_position=-1):
        A, Hq, _ = self.q.shape
        if mirror and A:
            max_position = int(self.pos_h.max())
        nbytes = pac.decode_workspace_size(self.cache, A, Hq, max_position, waves, kernel)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.q.device)
        hm = np.concatenate([self.pos_h, self.rows_h]) if mirror else None
        pac.decode_rope_store_attn(self.cache, 0, self.q, self.k_new, self.v_new, self.pos,
                                   self.rows, self.out, self.ws, self.cfg["base"],
                                   host_mirror=hm, status=self.status,
                                   waves=waves, kernel=kernel)
        torch.cuda.synchronize()
        return self.out


def oracle_rows(q, k_new, v_new, Kpre, Vpre, positions, rows, base, entries, dtype="bf16"):
    """Run the oracle entry by entry on a host copy of each row's prefix.

    Returns {a: (out[Hq, D] uint16, k_slot[Hkv, D] uint16, v_slot[Hkv, D] uint16)}.
    Kpre / Vpre: the cache BEFORE the step (torch, any device).
    """
    res = {}
    qb, kb, vb = workloads.bits(q), workloads.bits(k_new), workloads.bits(v_new)
    for a in entries:
        p, r = int(positions[a]), int(rows[a])
        Km = workloads.bits(Kpre[r, :p + 1]).reshape((1, p + 1) + tuple(Kpre.shape[2:])).copy()
        Vm = workloads.bits(Vpre[r, :p + 1]).reshape((1, p + 1) + tuple(Vpre.shape[2:])).copy()
        out = oracle.decode_step(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [p], [0], Km, Vm, base,
                                 dtype=dtype)
        res[a] = (out[0], Km[0, p].copy(), Vm[0, p].copy())
    return res


def check_output(got_bits, want_bits, what="", dtype="bf16"):
    g = widen(got_bits, dtype).astype(np.float64)
    w = widen(want_bits, dtype).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - w)
    mx, rms = float(err.max()), float(np.sqrt(np.mean(err ** 2)))
    log(f"  {what} ({dtype}): max-abs {mx:.3e} rms {rms:.3e} "
        f"exact {np.mean(got_bits == want_bits):.4f}")
    assert mx <= MAX_ABS, f"{what}: max-abs {mx} > {MAX_ABS}"
    assert rms <= RMS, f"{what}: rms {rms} > {RMS}"
    return mx, rms


def check_untouched(run, Kpre, Vpre, active_slots):
    """Every cache byte except the (row, pos) slots equals its value before the step."""
    Kx, Vx = Kpre.clone(), Vpre.clone()
    for r, p in active_slots:
        Kx[r, p] = run.Kc[r, p]
        Vx[r, p] = run.Vc[r, p]
    assert torch.equal(Kx.view(torch.int16), run.Kc.view(torch.int16)), "K bytes changed outside slots"
    assert torch.equal(Vx.view(torch.int16), run.Vc.view(torch.int16)), "V bytes changed outside slots"


def full_parity(run, Kpre, Vpre, entries=None):
    """Compare every entry (or a subset) of a finished decode step with the oracle."""
    A = run.q.shape[0]
    entries = range(A) if entries is None else entries
    want = oracle_rows(run.q, run.k_new, run.v_new, Kpre, Vpre, run.pos_h, run.rows_h,
                       run.cfg["base"], entries, dtype=run.dtype)
    out = workloads.bits(run.out)
    got_o, want_o, kd = [], [], []
    for a, (o, ks, vs) in want.items():
        p, r = int(run.pos_h[a]), int(run.rows_h[a])
        kgot = workloads.bits(run.Kc[r, p])
        vgot = workloads.bits(run.Vc[r, p])
        assert np.array_equal(vgot, vs), f"V store differs at entry {a}"
        d = ulp_dist(kgot, ks)
        assert d.max() <= 1, f"K store off by {d.max()} ulp at entry {a}"
        kd.append(d)
        got_o.append(out[a])
        want_o.append(o)
    kd = np.concatenate([x.ravel() for x in kd])
    log(f"  K store: exact fraction {np.mean(kd == 0):.6f}, max ulp {kd.max()}")
    return check_output(np.stack(got_o), np.stack(want_o), "output", dtype=run.dtype)


class _RawDevice:
    """A raw device address exposed through __cuda_array_interface__ (int16 elements)."""

    def __init__(self, ptr, nbytes):
        self.__cuda_array_interface__ = {"shape": (nbytes // 2,), "typestr": "<i2",
                                         "data": (int(ptr), False), "version": 3,
                                         "strides": None}


def _loaded_hip_runtime():
    import ctypes
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("HIP runtime not loaded")


def copy_to_device_ptr(ptr, src, nbytes):
    """Copy a host 16-bit tensor into raw device memory (test plumbing only)."""
    host = src.detach().contiguous().cpu().view(torch.int16).reshape(-1)
    assert host.numel() * 2 == nbytes
    try:
        dst = torch.as_tensor(_RawDevice(ptr, nbytes), device="cuda")
        dst.copy_(host)
    except Exception:  # noqa: BLE001 - torch without the interface: use the runtime itself
        import ctypes
        hip = _loaded_hip_runtime()
        rc = hip.hipMemcpy(ctypes.c_void_p(ptr), ctypes.c_void_p(host.data_ptr()),
                           ctypes.c_size_t(nbytes), 1)  # host to device
        assert rc == 0, rc
    torch.cuda.synchronize()
