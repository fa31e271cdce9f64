"""Seeded synthetic workloads for the positions-aware cached decode step.

This module only draws inputs.  It holds none of the method's arithmetic and
is the one piece of code that both the CPU oracle side (tests, CPU baseline)
and the HIP side (tests, bench) use.  Random tensor values come from torch's
generators (torch rounds its FP32 normal draws to BF16); positions and rows
from numpy's PCG64 generator.

Workload shapes follow the decode and prefill configurations the method is
measured on: a tiny case, a Llama-3-8B-like decode batch, a ragged
continuous batch with a long tail of positions, a long-context decode, an
equal-length batched prefill, and a chunked prefill of mixed starts and
lengths.  The pages measure on official model workloads
that are not available; these seeded draws stand in for them.
"""
import math

import numpy as np
import torch

# BF16 quiet-NaN pattern used to fill bytes that must never be read.
NAN_SENTINEL = 0x7FC1

CONFIGS = {
    # A=4 active rows in a 6-slot cache, capacity 128, H_q=4, H_kv=2, D=64.
    "tiny": dict(kind="decode", A=4, S=6, C=128, Hq=4, Hkv=2, D=64, base=1.0e4, sigma=1.0,
                 pos=("uniform", 0, 127), rows="subset", inactive="normal", seed=0),
    # Llama-3-8B-like decode: 64 rows in 64 slots, capacity 4096, 32/8/128.
    "llama3_8b": dict(kind="decode", A=64, S=64, C=4096, Hq=32, Hkv=8, D=128, base=5.0e5,
                      sigma=1.0, pos=("uniform", 1024, 4095), rows="identity",
                      inactive="normal", seed=1),
    # Ragged continuous batch: 200 survivors of 256 slots, capacity 8192,
    # positions log-uniform in [1, 8191]; inactive rows hold a NaN sentinel.
    "ragged": dict(kind="decode", A=200, S=256, C=8192, Hq=32, Hkv=8, D=128, base=5.0e5,
                   sigma=1.0, pos=("loguniform", 1, 8191), rows="subset", inactive="sentinel",
                   seed=2),
    # Long context: 8 rows, capacity 32768, H_q=64, H_kv=8, values N(0, 0.5).
    "long": dict(kind="decode", A=8, S=8, C=32768, Hq=64, Hkv=8, D=128, base=5.0e5, sigma=0.5,
                 pos=("uniform", 16384, 32767), rows="identity", inactive="normal", seed=3),
    # Equal-length batched prefill: 16 prompts of 1024 tokens into empty rows.
    "prefill": dict(kind="prefill", A=16, S=16, C=2048, T=1024, Hq=32, Hkv=8, D=128,
                    base=5.0e5, sigma=1.0, rows="identity", seed=4),
    # Chunked prefill with mixed lengths: 16 rows of a 4096-capacity cache,
    # each appending a chunk of 128..512 tokens (uniform) at a start uniform in
    # [0, 3072] (start 0: a fresh prompt), 32/8/128.
    "chunk": dict(kind="chunk", A=16, S=16, C=4096, T=512, Hq=32, Hkv=8, D=128, base=5.0e5,
                  sigma=1.0, starts=("uniform", 0, 3072), lens=("uniform", 128, 512),
                  rows="identity", seed=5),
}


# storage type of the 16-bit tensors: every config defaults to BF16; "f16"
# draws the same N(0, sigma) values rounded to FP16 instead
TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.setdefault("dtype", "bf16")
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def draw_indices(cfg):
    """positions[A] and cache_rows[A] (int32 numpy) for a decode config.

    uniform (lo, hi): integers uniform in [lo, hi].
    loguniform (lo, hi): floor(exp(u * ln(hi + 1))) clipped to [lo, hi], u ~ U[0, 1).
    rows 'identity': 0..A-1; 'subset': A distinct rows of S in random order.
    """
    rng = np.random.default_rng(cfg["seed"])
    A, S = cfg["A"], cfg["S"]
    if cfg["kind"] == "decode":
        kind, lo, hi = cfg["pos"]
        if kind == "uniform":
            pos = rng.integers(lo, hi + 1, size=A)
        elif kind == "loguniform":
            u = rng.random(size=A)
            pos = np.floor(np.exp(u * math.log(hi + 1))).astype(np.int64)
            pos = np.clip(pos, lo, hi)
        else:
            raise ValueError(kind)
    else:
        pos = np.zeros(A, dtype=np.int64)
    if cfg["rows"] == "identity":
        rows = np.arange(A)
    elif cfg["rows"] == "subset":
        rows = rng.permutation(S)[:A]
    else:
        raise ValueError(cfg["rows"])
    return pos.astype(np.int32), rows.astype(np.int32)


def draw_chunk_meta(cfg):
    """starts[A], lengths[A], rows[A] (int32 numpy) of a chunk config: starts
    and lengths uniform integers in their configured ranges (lengths clipped to
    T, starts to C - length); rows as in draw_indices."""
    rng = np.random.default_rng(cfg["seed"])
    A, S, C, T = cfg["A"], cfg["S"], cfg["C"], cfg["T"]
    _, lo, hi = cfg["lens"]
    lens = np.minimum(rng.integers(lo, hi + 1, size=A), T)
    _, lo, hi = cfg["starts"]
    starts = np.minimum(rng.integers(lo, hi + 1, size=A), C - lens)
    if cfg["rows"] == "identity":
        rows = np.arange(A)
    else:
        rows = rng.permutation(S)[:A]
    return starts.astype(np.int32), lens.astype(np.int32), rows.astype(np.int32)


def _normal(shape, gen, device, sigma, dtype="bf16", chunk_elems=1 << 28):
    """N(0, sigma) tensor drawn by torch in FP32 and rounded to the storage
    type (drawn in chunks along dim 0)."""
    out = torch.empty(shape, dtype=TORCH_DTYPES[dtype], device=device)
    flat = out.view(shape[0], -1)
    per = max(1, chunk_elems // max(1, flat.shape[1]))
    for i in range(0, shape[0], per):
        blk = torch.randn(flat[i:i + per].shape, generator=gen, device=device,
                          dtype=torch.float32)
        if sigma != 1.0:
            blk.mul_(sigma)
        flat[i:i + per].copy_(blk)
        del blk
    return out


def draw_decode(cfg, device="cpu"):
    """Inputs of one decode step as torch tensors on `device`.

    Returns dict with q [A,Hq,D], k_new/v_new [A,Hkv,D] (bf16), Kc/Vc
    [S,C,Hkv,D] (bf16 prior cache contents), positions/rows (int32 numpy).
    Inactive rows hold N(0, sigma) draws or the NaN sentinel, per config.
    """
    A, S, C, Hq, Hkv, D = (cfg[k] for k in ("A", "S", "C", "Hq", "Hkv", "D"))
    sigma = cfg.get("sigma", 1.0)
    pos, rows = draw_indices(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + cfg["seed"])
    q = _normal((A, Hq, D), gen, device, sigma, cfg["dtype"])
    k_new = _normal((A, Hkv, D), gen, device, sigma, cfg["dtype"])
    v_new = _normal((A, Hkv, D), gen, device, sigma, cfg["dtype"])
    Kc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
    Vc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
    if cfg.get("inactive") == "sentinel":
        inactive = np.setdiff1d(np.arange(S), rows)
        if inactive.size:
            idx = torch.as_tensor(inactive, device=device, dtype=torch.long)
            sent = torch.tensor(NAN_SENTINEL, dtype=torch.int16)
            Kc.view(torch.int16).index_fill_(0, idx, sent)
            Vc.view(torch.int16).index_fill_(0, idx, sent)
    return dict(q=q, k_new=k_new, v_new=v_new, Kc=Kc, Vc=Vc, positions=pos, rows=rows)


def draw_cache_layers(cfg, layers, device="cuda"):
    """Extra layer caches (K, V pairs) for a decode config, each [S, C, Hkv, D]
    N(0, sigma) BF16, seeded per layer; inactive rows get the sentinel if the
    config says so.  Used to rotate layers so a step does not re-read bytes a
    previous step left in the last-level cache."""
    S, C, Hkv, D = (cfg[k] for k in ("S", "C", "Hkv", "D"))
    sigma = cfg.get("sigma", 1.0)
    _, rows = draw_indices(cfg)
    out = []
    for l in range(layers):
        gen = torch.Generator(device=device)
        gen.manual_seed(5000 + 97 * cfg["seed"] + l)
        Kc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
        Vc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
        if cfg.get("inactive") == "sentinel":
            inactive = np.setdiff1d(np.arange(S), rows)
            if inactive.size:
                idx = torch.as_tensor(inactive, device=device, dtype=torch.long)
                sent = torch.tensor(NAN_SENTINEL, dtype=torch.int16)
                Kc.view(torch.int16).index_fill_(0, idx, sent)
                Vc.view(torch.int16).index_fill_(0, idx, sent)
        out.append((Kc, Vc))
    return out


def draw_prefill(cfg, device="cpu"):
    """Inputs of one prefill (or prefill chunk): q [A,T,Hq,D], k_new/v_new
    [A,T,Hkv,D], Kc/Vc [S,C,Hkv,D] with random prior bytes (for a chunk, the
    cached prefix before each start), rows (int32 numpy)."""
    A, S, C, T, Hq, Hkv, D = (cfg[k] for k in ("A", "S", "C", "T", "Hq", "Hkv", "D"))
    sigma = cfg.get("sigma", 1.0)
    if cfg["kind"] == "chunk":
        _, _, rows = draw_chunk_meta(cfg)
    else:
        _, rows = draw_indices(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed(2000 + cfg["seed"])
    q = _normal((A, T, Hq, D), gen, device, sigma, cfg["dtype"])
    k_new = _normal((A, T, Hkv, D), gen, device, sigma, cfg["dtype"])
    v_new = _normal((A, T, Hkv, D), gen, device, sigma, cfg["dtype"])
    Kc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
    Vc = _normal((S, C, Hkv, D), gen, device, sigma, cfg["dtype"])
    return dict(q=q, k_new=k_new, v_new=v_new, Kc=Kc, Vc=Vc, rows=rows)


def bits(t):
    """16-bit torch tensor (BF16 or FP16) -> numpy uint16 bit patterns (a host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(arr, device="cpu"):
    """numpy uint16 BF16 bit patterns -> BF16 torch tensor on device."""
    a = np.ascontiguousarray(arr, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
