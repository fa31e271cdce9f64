"""Pins of the CPU oracle against facts fixed outside it.

Each pin takes a loaded oracle (`oracle.Oracle`) and raises AssertionError
(or OracleError) when the oracle disagrees with what the pages or the
mathematics fix: hand values from closed forms, invariants of RoPE and of
softmax attention, special cases that reduce to textbook results, and brute
force in float64 (numpy, and torch's scaled_dot_product_attention on the CPU).

The same pins run against deliberately broken builds of the oracle in
test_oracle_pins.py, to show that a plausible mistake fails at least one.
"""
import math
import os

import numpy as np
import torch

import workloads
from bf16util import (bf16_exact, bf16_rne_f64, bf16_rne_f64_array, f16_rne_f64_array,
                      f16_to_f32, rope_f64, to_f32, ulp_dist)
from oracle import OracleError

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _empty_case(A, S, C, Hq, Hkv, D, seed=0):
    rng = np.random.default_rng(seed)
    def bf(shape):
        return workloads.bits(torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
                              .to(torch.bfloat16))
    return dict(q=bf((A, Hq, D)), k_new=bf((A, Hkv, D)), v_new=bf((A, Hkv, D)),
                Kc=bf((S, C, Hkv, D)), Vc=bf((S, C, Hkv, D)))


def _tiny():
    cfg = workloads.config("tiny")
    t = workloads.draw_decode(cfg, device="cpu")
    return cfg, dict(q=workloads.bits(t["q"]), k_new=workloads.bits(t["k_new"]),
                     v_new=workloads.bits(t["v_new"]), Kc=workloads.bits(t["Kc"]),
                     Vc=workloads.bits(t["Vc"]), positions=t["positions"], rows=t["rows"])


# --------------------------------------------------------------------------- RoPE

def pin_bf16_rounding(orc):
    """Round-to-nearest-even FP32 -> BF16 on ties, carries, NaN and infinities."""
    cases = {1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000}
    for v, b in cases.items():
        assert orc.f32_to_bf16(v) == b
    f = lambda u: np.array([u], dtype=np.uint32).view(np.float32)[0]
    assert orc.f32_to_bf16(f(0x3F808000)) == 0x3F80      # tie, even stays
    assert orc.f32_to_bf16(f(0x3F818000)) == 0x3F82      # tie, odd rounds up
    assert orc.f32_to_bf16(f(0x3F808001)) == 0x3F81      # above tie
    assert orc.f32_to_bf16(f(0x3F807FFF)) == 0x3F80      # below tie
    assert orc.f32_to_bf16(f(0x3FFF8000)) == 0x4000      # carry into exponent
    assert orc.f32_to_bf16(f(0x7F7FFFFF)) == 0x7F80      # overflow to infinity
    assert orc.f32_to_bf16(float("inf")) == 0x7F80
    nan = orc.f32_to_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    rng = np.random.default_rng(5)
    xs = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(x) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _store_one(orc, k_vec, pos, base, D, Hkv=1, Hq=1):
    """Run a one-entry decode and return the stored K slot (row 1 of 2, head 0)."""
    C = max(8, pos + 1)
    Kc = np.zeros((2, C, Hkv, D), dtype=np.uint16)
    Vc = np.zeros((2, C, Hkv, D), dtype=np.uint16)
    k = np.zeros((1, Hkv, D), dtype=np.uint16)
    k[0, 0] = k_vec
    q = np.zeros((1, Hq, D), dtype=np.uint16)
    v = np.zeros((1, Hkv, D), dtype=np.uint16)
    orc.decode_step(q, k, v, [pos], [1], Kc, Vc, base)
    return Kc[1, pos, 0]


def pin_rope_hand_values(orc):
    """Hand values of split-half RoPE from the closed form cos/sin at known angles.

    D=64, base 1e4: unit vector e_0 at pos 1 has angle 1 rad, so the stored pair
    (0, 32) is (bf16(cos 1), bf16(sin 1)) = (0x3F0A, 0x3F57); e_1 at pos 3 uses
    inv_freq_1 = 1e4^(-1/32); x = y = 1 at pos 5 gives (cos5 - sin5, sin5 + cos5).
    D=128, base 5e5 at positions 4095 and 32767 (where the FP32 angle matters).
    """
    one = bf16_exact(1.0)
    cases = []
    with open(os.path.join(GOLDEN, "rope_hand_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                D, base, pos, i, x, y = (int(float(v)) for v in line[:6])
                cases.append((D, float(base), pos, i, x, y, int(line[6], 16), int(line[7], 16)))
    assert len(cases) == 6
    for D, base, pos, i, x, y, lo_b, hi_b in cases:
        k = np.zeros(D, dtype=np.uint16)
        if x:
            k[i] = one
        if y:
            k[i + D // 2] = one
        got = _store_one(orc, k, pos, base, D)
        assert got[i] == lo_b, (D, pos, i, hex(got[i]), hex(lo_b))
        assert got[i + D // 2] == hi_b, (D, pos, i, hex(got[i + D // 2]), hex(hi_b))
        other = np.delete(got, [i, i + D // 2])
        assert np.all((other & 0x7FFF) == 0), "a unit pair leaked into other elements"
        # the same numbers from float64 closed form (the FP32 angle is exact here
        # when inv_freq is 1, i.e. i = 0)
        if i == 0:
            th = float(pos)
            lo = x * math.cos(th) - y * math.sin(th)
            hi = y * math.cos(th) + x * math.sin(th)
            assert abs(int(bf16_rne_f64(lo)) - lo_b) <= 1 and abs(int(bf16_rne_f64(hi)) - hi_b) <= 1


def pin_rope_identity_at_zero(orc):
    """At position 0 every angle is 0: the stored K equals k_new bit for bit."""
    rng = np.random.default_rng(1)
    D = 64
    k = workloads.bits(torch.from_numpy(rng.standard_normal(D).astype(np.float32))
                       .to(torch.bfloat16))
    got = _store_one(orc, k, 0, 1e4, D)
    assert np.array_equal(got, k)


def pin_rope_norm(orc):
    """RoPE preserves every pair's norm (before BF16 rounding), to FP32 rounding."""
    rng = np.random.default_rng(2)
    for D, base, pos in [(64, 1e4, 7), (128, 5e5, 4095), (128, 5e5, 32767)]:
        x = rng.standard_normal(D).astype(np.float32)
        y = orc.rope_apply(x, pos, base)
        h = D // 2
        n0 = x[:h].astype(np.float64) ** 2 + x[h:].astype(np.float64) ** 2
        n1 = y[:h].astype(np.float64) ** 2 + y[h:].astype(np.float64) ** 2
        assert np.allclose(n1, n0, rtol=4e-7 * 8, atol=1e-12)
        assert not np.allclose(y, x)  # it did rotate


def pin_rope_vs_f64(orc):
    """The FP32 rotation agrees with the float64 closed form to FP32 angle error."""
    rng = np.random.default_rng(3)
    for D, base, pos in [(64, 1e4, 1), (64, 1e4, 100), (128, 5e5, 4000), (128, 5e5, 30000)]:
        x = rng.standard_normal(D).astype(np.float32)
        y = orc.rope_apply(x, pos, base).astype(np.float64)
        ref = rope_f64(x.astype(np.float64), pos, base)
        # fl32(pos * inv_freq) differs from the exact angle by <= pos * 2^-23 rad
        tol = 4.0 * (pos * 2.0 ** -23 + 2.0 ** -23) * np.abs(x).max() + 1e-6
        assert np.abs(y - ref).max() <= tol, (D, pos, np.abs(y - ref).max(), tol)


def pin_rope_relative(orc):
    """q'_m . k'_n depends only on m - n: shifting both positions keeps the score."""
    rng = np.random.default_rng(4)
    D, base = 64, 1e4
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    for m, n, c in [(5, 2, 10), (40, 0, 57), (3, 3, 100)]:
        s0 = float(np.dot(orc.rope_apply(q, m, base).astype(np.float64),
                          orc.rope_apply(k, n, base).astype(np.float64)))
        s1 = float(np.dot(orc.rope_apply(q, m + c, base).astype(np.float64),
                          orc.rope_apply(k, n + c, base).astype(np.float64)))
        assert abs(s0 - s1) <= 2e-4 * np.linalg.norm(q) * np.linalg.norm(k), (m, n, c, s0, s1)


# ----------------------------------------------------------------- attention

def pin_single_key(orc):
    """pos = 0: one key, softmax weight 1, the output is v_new of the kv head, bit for bit."""
    A, S, C, Hq, Hkv, D = 3, 4, 16, 8, 2, 64
    c = _empty_case(A, S, C, Hq, Hkv, D, seed=7)
    out = orc.decode_step(c["q"], c["k_new"], c["v_new"], [0, 0, 0], [3, 0, 2], c["Kc"], c["Vc"],
                          1e4)
    G = Hq // Hkv
    for a in range(A):
        for hq in range(Hq):
            assert np.array_equal(out[a, hq], c["v_new"][a, hq // G])


def pin_uniform_softmax(orc):
    """q = 0 gives equal weights: the output is the mean of V over keys 0..pos.

    V rows 1, 2 and (new token) 4 at pos 2: mean 7/3 -> BF16 0x4015.
    """
    D = 64
    Kc = np.zeros((1, 4, 1, D), dtype=np.uint16)
    Vc = np.zeros((1, 4, 1, D), dtype=np.uint16)
    Vc[0, 0, 0, :] = bf16_exact(1.0)
    Vc[0, 1, 0, :] = bf16_exact(2.0)
    v = np.full((1, 1, D), bf16_exact(4.0), dtype=np.uint16)
    k = np.zeros((1, 1, D), dtype=np.uint16)
    q = np.zeros((1, 1, D), dtype=np.uint16)
    out = orc.decode_step(q, k, v, [2], [0], Kc, Vc, 1e4)
    assert np.all(out == 0x4015)
    # random V: mean to one BF16 ulp of the float64 mean
    rng = np.random.default_rng(8)
    S, C, Hkv, Hq, A = 3, 50, 2, 4, 3
    cs = _empty_case(A, S, C, Hq, Hkv, D, seed=9)
    pos = np.array([10, 49, 0], dtype=np.int32)
    rows = np.array([2, 0, 1], dtype=np.int32)
    q = np.zeros((A, Hq, D), dtype=np.uint16)
    out = orc.decode_step(q, cs["k_new"], cs["v_new"], pos, rows, cs["Kc"], cs["Vc"], 1e4)
    G = Hq // Hkv
    for a in range(A):
        for hq in range(Hq):
            vals = to_f32(cs["Vc"][rows[a], :pos[a] + 1, hq // G]).astype(np.float64)
            ref = bf16_rne_f64_array(vals.mean(axis=0))
            assert ulp_dist(out[a, hq], ref).max() <= 1
    del rng


def pin_constant_v(orc):
    """All values equal c: output c (exact for a power of two, else <= 1 ulp)."""
    A, S, C, Hq, Hkv, D = 2, 3, 40, 4, 1, 64
    cs = _empty_case(A, S, C, Hq, Hkv, D, seed=10)
    for cval, tol in [(2.0, 0), (1.5, 1), (-0.375, 0)]:
        Vc = np.full_like(cs["Vc"], bf16_exact(cval))
        v = np.full_like(cs["v_new"], bf16_exact(cval))
        Kc = cs["Kc"].copy()
        out = orc.decode_step(cs["q"], cs["k_new"], v, [39, 17], [2, 0], Kc, Vc, 1e4)
        assert ulp_dist(out, np.full_like(out, bf16_exact(cval))).max() <= tol


def pin_dominant_key(orc):
    """A key whose score exceeds every other by >= 30 takes all the weight.

    (a) the new token: q = k_new = 16 on four coordinates; its rotated self-dot
        is 1024 while all cached keys are 0, so out = v_new exactly;
    (b) a cached key j* equal to the float64-rotated query, rounded to BF16.
    """
    D, C = 64, 32
    q = np.zeros((1, 1, D), dtype=np.uint16)
    q[0, 0, :4] = bf16_exact(16.0)
    Kc = np.zeros((1, C, 1, D), dtype=np.uint16)
    rng = np.random.default_rng(11)
    Vc = workloads.bits(torch.from_numpy(rng.standard_normal((1, C, 1, D)).astype(np.float32))
                        .to(torch.bfloat16))
    v = Vc[0, 0:1].copy() ^ 0  # any values
    v[0, 0, :] = bf16_exact(3.25)
    out = orc.decode_step(q, q.copy(), v, [20], [0], Kc.copy(), Vc.copy(), 1e4)
    assert np.all(out == bf16_exact(3.25))
    # (b)
    pos, jstar = 20, 7
    qrot = rope_f64(to_f32(q[0, 0]).astype(np.float64), pos, 1e4)
    Kc2 = np.zeros((1, C, 1, D), dtype=np.uint16)
    Kc2[0, jstar, 0] = bf16_rne_f64_array(qrot)
    k_new = np.zeros((1, 1, D), dtype=np.uint16)
    out = orc.decode_step(q, k_new, v, [pos], [0], Kc2, Vc.copy(), 1e4)
    assert ulp_dist(out[0, 0], Vc[0, jstar, 0]).max() <= 1


def _ref_attention_f64(q_bits, Kc, Vc, positions, rows, base, G):
    """float64 attention over the (already updated) cache: the definition, as loops."""
    A, Hq, D = q_bits.shape
    out = np.zeros((A, Hq, D))
    for a in range(A):
        p, r = int(positions[a]), int(rows[a])
        for hq in range(Hq):
            qr = rope_f64(to_f32(q_bits[a, hq]).astype(np.float64), p, base)
            K = to_f32(Kc[r, :p + 1, hq // G]).astype(np.float64)
            V = to_f32(Vc[r, :p + 1, hq // G]).astype(np.float64)
            s = K @ qr / math.sqrt(D)
            w = np.exp(s - s.max())
            out[a, hq] = (w @ V) / w.sum()
    return out


def pin_brute_force_f64(orc):
    """Tiny decode config vs float64 brute force: K store within 1 ulp of the
    float64 rotation, V store bit-exact, output within 1 ulp of the float64 truth,
    and the same through torch's scaled_dot_product_attention (float64, CPU) on
    repeat-interleaved K/V."""
    cfg, c = _tiny()
    Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
    out = orc.decode_step(c["q"], c["k_new"], c["v_new"], c["positions"], c["rows"], Kc, Vc,
                          cfg["base"])
    G = cfg["Hq"] // cfg["Hkv"]
    for a in range(cfg["A"]):
        p, r = c["positions"][a], c["rows"][a]
        kref = bf16_rne_f64_array(rope_f64(to_f32(c["k_new"][a]).astype(np.float64), p,
                                           cfg["base"]))
        assert ulp_dist(Kc[r, p], kref).max() <= 1
        assert np.array_equal(Vc[r, p], c["v_new"][a])
    ref = _ref_attention_f64(c["q"], Kc, Vc, c["positions"], c["rows"], cfg["base"], G)
    assert ulp_dist(out, bf16_rne_f64_array(ref)).max() <= 1
    # library cross-check: SDPA in float64
    for a in range(cfg["A"]):
        p, r = int(c["positions"][a]), int(c["rows"][a])
        qr = np.stack([rope_f64(to_f32(c["q"][a, h]).astype(np.float64), p, cfg["base"])
                       for h in range(cfg["Hq"])])
        K = torch.from_numpy(to_f32(Kc[r, :p + 1]).astype(np.float64)).permute(1, 0, 2)
        V = torch.from_numpy(to_f32(Vc[r, :p + 1]).astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr)[:, None, :], K, V)[:, 0, :].numpy()
        assert ulp_dist(out[a], bf16_rne_f64_array(o)).max() <= 1


def pin_gqa_equals_mha(orc):
    """GQA equals MHA on K/V heads repeated G times (kv head = hq / G)."""
    A, S, C, Hq, Hkv, D = 3, 4, 24, 8, 2, 64
    G = Hq // Hkv
    c = _empty_case(A, S, C, Hq, Hkv, D, seed=12)
    pos, rows = [5, 23, 11], [1, 3, 0]
    Kg, Vg = c["Kc"].copy(), c["Vc"].copy()
    out_g = orc.decode_step(c["q"], c["k_new"], c["v_new"], pos, rows, Kg, Vg, 1e4)
    Km = np.ascontiguousarray(np.repeat(c["Kc"], G, axis=2))
    Vm = np.ascontiguousarray(np.repeat(c["Vc"], G, axis=2))
    out_m = orc.decode_step(c["q"], np.repeat(c["k_new"], G, axis=1),
                            np.repeat(c["v_new"], G, axis=1), pos, rows, Km, Vm, 1e4)
    assert np.array_equal(out_g, out_m)


def pin_untouched_and_sentinel(orc):
    """Only slots (rows[a], pos[a]) change; NaN sentinels in inactive rows and
    beyond each prefix are never read (output finite and unchanged)."""
    cfg, c = _tiny()
    Kc0, Vc0 = c["Kc"].copy(), c["Vc"].copy()
    Kc, Vc = Kc0.copy(), Vc0.copy()
    out = orc.decode_step(c["q"], c["k_new"], c["v_new"], c["positions"], c["rows"], Kc, Vc,
                          cfg["base"])
    mask = np.ones(Kc.shape[:2], dtype=bool)
    for p, r in zip(c["positions"], c["rows"]):
        mask[r, p] = False
    assert np.array_equal(Kc[mask], Kc0[mask]) and np.array_equal(Vc[mask], Vc0[mask])
    # poison everything that must not be read
    Kp, Vp = Kc0.copy(), Vc0.copy()
    poison = np.ones(Kc.shape[:2], dtype=bool)
    for p, r in zip(c["positions"], c["rows"]):
        poison[r, :p] = False
    Kp[poison] = workloads.NAN_SENTINEL
    Vp[poison] = workloads.NAN_SENTINEL
    out2 = orc.decode_step(c["q"], c["k_new"], c["v_new"], c["positions"], c["rows"], Kp, Vp,
                           cfg["base"])
    assert np.all(np.isfinite(to_f32(out2)))
    assert np.array_equal(out, out2)


def pin_idempotent_and_permutation(orc):
    """Running the step twice equals once; permuting entries permutes outputs."""
    cfg, c = _tiny()
    K1, V1 = c["Kc"].copy(), c["Vc"].copy()
    o1 = orc.decode_step(c["q"], c["k_new"], c["v_new"], c["positions"], c["rows"], K1, V1,
                         cfg["base"])
    K2, V2 = K1.copy(), V1.copy()
    o2 = orc.decode_step(c["q"], c["k_new"], c["v_new"], c["positions"], c["rows"], K2, V2,
                         cfg["base"])
    assert np.array_equal(o1, o2) and np.array_equal(K1, K2) and np.array_equal(V1, V2)
    perm = np.array([2, 0, 3, 1])
    K3, V3 = c["Kc"].copy(), c["Vc"].copy()
    o3 = orc.decode_step(c["q"][perm], c["k_new"][perm], c["v_new"][perm], c["positions"][perm],
                         c["rows"][perm], K3, V3, cfg["base"])
    assert np.array_equal(o3, o1[perm]) and np.array_equal(K3, K1) and np.array_equal(V3, V1)


def pin_errors(orc):
    """Invalid indices fail explicitly and write nothing."""
    cfg, c = _tiny()
    for pos, rows in [([1, 2, 3, 4], [0, 1, 1, 2]),      # duplicate row
                      ([1, 2, 3, 128], [0, 1, 2, 3]),    # position out of range
                      ([1, 2, 3, -1], [0, 1, 2, 3]),
                      ([1, 2, 3, 4], [0, 1, 2, 6])]:     # row out of range
        Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
        try:
            orc.decode_step(c["q"], c["k_new"], c["v_new"], pos, rows, Kc, Vc, cfg["base"])
        except OracleError:
            pass
        else:
            raise AssertionError(f"accepted invalid indices {pos} {rows}")
        assert np.array_equal(Kc, c["Kc"]) and np.array_equal(Vc, c["Vc"])


# ------------------------------------------------------------------- prefill

def _prefill_case(A, T, S, C, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    def bf(shape):
        return workloads.bits(torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
                              .to(torch.bfloat16))
    return dict(q=bf((A, T, Hq, D)), k=bf((A, T, Hkv, D)), v=bf((A, T, Hkv, D)),
                Kc=bf((S, C, Hkv, D)), Vc=bf((S, C, Hkv, D)))


def pin_prefill_brute_force(orc):
    """Prefill vs float64 causal SDPA on repeat-interleaved K/V after float64 RoPE;
    stores within 1 ulp (K) / exact (V); positions >= T and other rows untouched."""
    A, T, S, C, Hq, Hkv, D, base = 2, 13, 3, 20, 4, 2, 64, 1e4
    G = Hq // Hkv
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=13)
    rows = np.array([2, 0], dtype=np.int32)
    Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
    out = orc.prefill(c["q"], c["k"], c["v"], rows, Kc, Vc, base)
    untouched = np.ones((S, C), dtype=bool)
    for a in range(A):
        r = rows[a]
        untouched[r, :T] = False
        for t in range(T):
            kref = bf16_rne_f64_array(rope_f64(to_f32(c["k"][a, t]).astype(np.float64), t, base))
            assert ulp_dist(Kc[r, t], kref).max() <= 1
        assert np.array_equal(Vc[r, :T], c["v"][a])
        qr = np.stack([rope_f64(to_f32(c["q"][a, t]).astype(np.float64), t, base)
                       for t in range(T)])                      # [T, Hq, D]
        K = torch.from_numpy(to_f32(Kc[r, :T]).astype(np.float64)).permute(1, 0, 2)
        V = torch.from_numpy(to_f32(Vc[r, :T]).astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr).permute(1, 0, 2).contiguous(), K, V, is_causal=True)
        o = o.permute(1, 0, 2).numpy()
        assert ulp_dist(out[a], bf16_rne_f64_array(o)).max() <= 1
    assert np.array_equal(Kc[untouched], c["Kc"][untouched])
    assert np.array_equal(Vc[untouched], c["Vc"][untouched])


def pin_decode_after_prefill(orc):
    """Prefill of T tokens then a decode at position T equals the last query of a
    prefill of T + 1 tokens (bit for bit: the same definition either way)."""
    A, T, S, C, Hq, Hkv, D, base = 2, 9, 2, 16, 4, 2, 32, 1e4
    c = _prefill_case(A, T + 1, S, C, Hq, Hkv, D, seed=14)
    rows = np.array([1, 0], dtype=np.int32)
    K1, V1 = c["Kc"].copy(), c["Vc"].copy()
    full = orc.prefill(c["q"], c["k"], c["v"], rows, K1, V1, base)
    K2, V2 = c["Kc"].copy(), c["Vc"].copy()
    orc.prefill(c["q"][:, :T], c["k"][:, :T], c["v"][:, :T], rows, K2, V2, base)
    dec = orc.decode_step(c["q"][:, T], c["k"][:, T], c["v"][:, T], [T, T], rows, K2, V2, base)
    assert np.array_equal(dec, full[:, T])
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2)


def pin_prefill_subset(orc):
    """Computing a subset of query positions gives the same values as all of them."""
    A, T, S, C, Hq, Hkv, D, base = 1, 12, 1, 12, 2, 1, 16, 1e4
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=15)
    full = orc.prefill(c["q"], c["k"], c["v"], [0], c["Kc"].copy(), c["Vc"].copy(), base)
    sub = orc.prefill(c["q"], c["k"], c["v"], [0], c["Kc"].copy(), c["Vc"].copy(), base,
                      t_list=[0, 5, 11])
    assert np.array_equal(sub[:, [0, 5, 11]], full[:, [0, 5, 11]])


def pin_chunk_brute_force(orc):
    """A chunk appended at nonzero per-entry starts over a random cached prefix,
    vs float64 causal attention written out: token t of entry a is rotated at
    s_a + t (K within 1 ulp of the float64 rotation, V exact), query t attends
    slots 0 .. s_a + t of its row (output within 1 ulp of the float64 truth, and
    of SDPA with an explicit boolean mask); slots outside s_a .. s_a+T-1 and
    other rows untouched."""
    A, T, S, C, Hq, Hkv, D, base = 3, 7, 4, 24, 4, 2, 32, 1e4
    G = Hq // Hkv
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=16)
    rows = np.array([3, 0, 1], dtype=np.int32)
    starts = np.array([5, 0, 17], dtype=np.int32)            # 17 + 7 == C: full row
    Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
    out = orc.prefill(c["q"], c["k"], c["v"], rows, Kc, Vc, base, starts=starts)
    untouched = np.ones((S, C), dtype=bool)
    for a in range(A):
        r, s0 = rows[a], int(starts[a])
        untouched[r, s0:s0 + T] = False
        for t in range(T):
            kref = bf16_rne_f64_array(rope_f64(to_f32(c["k"][a, t]).astype(np.float64),
                                               s0 + t, base))
            assert ulp_dist(Kc[r, s0 + t], kref).max() <= 1
        assert np.array_equal(Vc[r, s0:s0 + T], c["v"][a])
        n = s0 + T
        K = to_f32(Kc[r, :n]).astype(np.float64)               # [n, Hkv, D]
        V = to_f32(Vc[r, :n]).astype(np.float64)
        ref = np.zeros((T, Hq, D))
        for t in range(T):
            for hq in range(Hq):
                qr = rope_f64(to_f32(c["q"][a, t, hq]).astype(np.float64), s0 + t, base)
                sc = K[:s0 + t + 1, hq // G] @ qr / math.sqrt(D)
                w = np.exp(sc - sc.max())
                ref[t, hq] = (w @ V[:s0 + t + 1, hq // G]) / w.sum()
        assert ulp_dist(out[a], bf16_rne_f64_array(ref)).max() <= 1
        qr = np.stack([rope_f64(to_f32(c["q"][a, t]).astype(np.float64), s0 + t, base)
                       for t in range(T)])                      # [T, Hq, D]
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        mask = torch.arange(n)[None, :] <= (s0 + torch.arange(T))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr).permute(1, 0, 2).contiguous(), Kt, Vt, attn_mask=mask)
        assert ulp_dist(out[a], bf16_rne_f64_array(o.permute(1, 0, 2).numpy())).max() <= 1
    assert np.array_equal(Kc[untouched], c["Kc"][untouched])
    assert np.array_equal(Vc[untouched], c["Vc"][untouched])


def pin_chunk_is_decode_steps(orc):
    """A chunk of T tokens at start s equals T decode steps at positions
    s .. s+T-1 (outputs and cache bit for bit), and splitting a chunk in two
    changes nothing."""
    A, T, S, C, Hq, Hkv, D, base = 2, 6, 3, 20, 4, 1, 16, 1e4
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=17)
    rows = np.array([2, 1], dtype=np.int32)
    starts = np.array([9, 3], dtype=np.int32)
    K1, V1 = c["Kc"].copy(), c["Vc"].copy()
    whole = orc.prefill(c["q"], c["k"], c["v"], rows, K1, V1, base, starts=starts)
    K2, V2 = c["Kc"].copy(), c["Vc"].copy()
    for t in range(T):
        dec = orc.decode_step(c["q"][:, t], c["k"][:, t], c["v"][:, t], starts + t, rows,
                              K2, V2, base)
        assert np.array_equal(dec, whole[:, t])
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2)
    K3, V3 = c["Kc"].copy(), c["Vc"].copy()
    h = 4
    o1 = orc.prefill(c["q"][:, :h], c["k"][:, :h], c["v"][:, :h], rows, K3, V3, base,
                     starts=starts)
    o2 = orc.prefill(c["q"][:, h:], c["k"][:, h:], c["v"][:, h:], rows, K3, V3, base,
                     starts=starts + h)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), whole)
    assert np.array_equal(K1, K3) and np.array_equal(V1, V3)


def pin_ragged_groups(orc):
    """A batch whose entries have different lengths equals the equal-length
    groups run one after another, bit for bit; tokens past an entry's length
    are neither stored nor attended and their output rows are not written."""
    A, T, S, C, Hq, Hkv, D, base = 3, 9, 4, 24, 4, 2, 16, 1e4
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=19)
    rows = np.array([1, 3, 0], dtype=np.int32)
    starts = np.array([4, 0, 15], dtype=np.int32)
    lens = np.array([9, 2, 5], dtype=np.int32)
    Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
    sentinel = np.full((A, T, Hq, D), 0x7fc1, dtype=np.uint16)
    out = orc.prefill(c["q"], c["k"], c["v"], rows, Kc, Vc, base, starts=starts, lens=lens,
                      out=sentinel.copy())
    K1, V1 = c["Kc"].copy(), c["Vc"].copy()
    for a in range(A):
        n = int(lens[a])
        o = orc.prefill(c["q"][a:a + 1, :n], c["k"][a:a + 1, :n], c["v"][a:a + 1, :n],
                        rows[a:a + 1], K1, V1, base, starts=starts[a:a + 1])
        assert np.array_equal(out[a, :n], o[0])
        assert np.array_equal(out[a, n:], sentinel[a, n:])
    assert np.array_equal(Kc, K1) and np.array_equal(Vc, V1)
    touched = np.zeros((S, C), dtype=bool)
    for a in range(A):
        touched[rows[a], starts[a]:starts[a] + lens[a]] = True
    assert np.array_equal(Kc[~touched], c["Kc"][~touched])
    assert np.array_equal(Vc[~touched], c["Vc"][~touched])
    assert not np.array_equal(Kc[touched], c["Kc"][touched])


def pin_chunk_errors(orc):
    """A chunk that would run past the row's capacity, or a negative start,
    fails explicitly and writes nothing; start 0 is the plain prefill."""
    A, T, S, C, Hq, Hkv, D, base = 2, 5, 2, 12, 2, 1, 16, 1e4
    c = _prefill_case(A, T, S, C, Hq, Hkv, D, seed=18)
    rows = [0, 1]
    for starts, lens in (([8, 0], None), ([-1, 0], None), ([12, 3], None), ([0, 0], [0, 5]),
                         ([0, 0], [6, 5]), ([9, 0], [4, 5])):
        Kc, Vc = c["Kc"].copy(), c["Vc"].copy()
        try:
            orc.prefill(c["q"], c["k"], c["v"], rows, Kc, Vc, base, starts=starts, lens=lens)
        except OracleError:
            pass
        else:
            raise AssertionError(f"accepted starts {starts} lens {lens}")
        assert np.array_equal(Kc, c["Kc"]) and np.array_equal(Vc, c["Vc"])
    a = orc.prefill(c["q"], c["k"], c["v"], rows, c["Kc"].copy(), c["Vc"].copy(), base,
                    starts=[0, 0])
    b = orc.prefill(c["q"], c["k"], c["v"], rows, c["Kc"].copy(), c["Vc"].copy(), base)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------- FP16

def pin_f16_rounding(orc):
    """FP16 conversions: the hand values of tests/golden/f16_hand_values.txt
    (binary16 definition), every one of the 65536 codes widened exactly as
    numpy's float16 does, and random FP32 values over the whole FP16 range
    (subnormals and overflow included) narrowed as numpy rounds them."""
    with open(os.path.join(GOLDEN, "f16_hand_values.txt")) as f:
        for line in f:
            cols = line.split("#")[0].split()
            if not cols:
                continue
            x = np.float32(float(cols[0]))
            assert float(x) == float(cols[0]), cols[0]
            assert orc.f32_to_f16(x) == int(cols[1], 16), cols
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(c)) for c in codes], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(6)
    xs = (rng.uniform(-1.0, 1.0, 40000) * 2.0 ** rng.integers(-27, 18, 40000)).astype(np.float32)
    # exact ties: codes' midpoints (from neighbouring FP16 values, exact in FP32)
    lo = rng.integers(0, 0x7BFF, 4000).astype(np.uint16)
    mid = ((lo.view(np.float16).astype(np.float64) +
            (lo + 1).astype(np.uint16).view(np.float16).astype(np.float64)) / 2).astype(np.float32)
    xs = np.concatenate([xs, mid, -mid, np.float32([np.inf, -np.inf])])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(x) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)
    q = orc.f32_to_f16(float("nan"))
    assert (q & 0x7C00) == 0x7C00 and (q & 0x3FF) != 0


def _f16_case(shape, rng, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float16).view(np.uint16)


def pin_f16_decode_brute_force(orc):
    """Decode with FP16 storage vs float64: K store within 1 FP16 ulp of the
    float64 rotation, V bit-exact, output within 1 ulp of the float64 truth;
    other rows untouched."""
    A, S, C, Hq, Hkv, D, base = 3, 5, 40, 4, 2, 64, 1e4
    G = Hq // Hkv
    rng = np.random.default_rng(21)
    q, k, v = _f16_case((A, Hq, D), rng), _f16_case((A, Hkv, D), rng), _f16_case((A, Hkv, D), rng)
    K0, V0 = _f16_case((S, C, Hkv, D), rng), _f16_case((S, C, Hkv, D), rng)
    pos = np.array([0, 17, 39], dtype=np.int32)
    rows = np.array([4, 1, 2], dtype=np.int32)
    Kc, Vc = K0.copy(), V0.copy()
    out = orc.decode_step(q, k, v, pos, rows, Kc, Vc, base, dtype="f16")
    touched = np.zeros((S, C), dtype=bool)
    for a in range(A):
        p_, r = int(pos[a]), int(rows[a])
        touched[r, p_] = True
        kref = f16_rne_f64_array(rope_f64(f16_to_f32(k[a]).astype(np.float64), p_, base))
        assert ulp_dist(Kc[r, p_], kref).max() <= 1
        assert np.array_equal(Vc[r, p_], v[a])
        Kf = f16_to_f32(Kc[r, :p_ + 1]).astype(np.float64)
        Vf = f16_to_f32(Vc[r, :p_ + 1]).astype(np.float64)
        for hq in range(Hq):
            qr = rope_f64(f16_to_f32(q[a, hq]).astype(np.float64), p_, base)
            sc = Kf[:, hq // G] @ qr / math.sqrt(D)
            w = np.exp(sc - sc.max())
            o = (w @ Vf[:, hq // G]) / w.sum()
            assert ulp_dist(out[a, hq], f16_rne_f64_array(o)).max() <= 1
    assert np.array_equal(Kc[~touched], K0[~touched]) and np.array_equal(Vc[~touched], V0[~touched])


def pin_f16_chunk_brute_force(orc):
    """Prefill chunk with FP16 storage at two nonzero starts vs float64 causal
    attention over the cached prefix and the chunk."""
    A, T, S, C, Hq, Hkv, D, base = 2, 6, 3, 20, 4, 1, 32, 1e4
    rng = np.random.default_rng(22)
    q, k, v = (_f16_case((A, T, Hq, D), rng), _f16_case((A, T, Hkv, D), rng),
               _f16_case((A, T, Hkv, D), rng))
    K0, V0 = _f16_case((S, C, Hkv, D), rng), _f16_case((S, C, Hkv, D), rng)
    rows = np.array([2, 0], dtype=np.int32)
    starts = np.array([3, 14], dtype=np.int32)
    Kc, Vc = K0.copy(), V0.copy()
    out = orc.prefill(q, k, v, rows, Kc, Vc, base, starts=starts, dtype="f16")
    for a in range(A):
        r, s0 = int(rows[a]), int(starts[a])
        for t in range(T):
            kref = f16_rne_f64_array(rope_f64(f16_to_f32(k[a, t]).astype(np.float64), s0 + t, base))
            assert ulp_dist(Kc[r, s0 + t], kref).max() <= 1
        assert np.array_equal(Vc[r, s0:s0 + T], v[a])
        Kf = f16_to_f32(Kc[r]).astype(np.float64)
        Vf = f16_to_f32(Vc[r]).astype(np.float64)
        for t in range(T):
            for hq in range(Hq):
                qr = rope_f64(f16_to_f32(q[a, t, hq]).astype(np.float64), s0 + t, base)
                sc = Kf[:s0 + t + 1, 0] @ qr / math.sqrt(D)
                w = np.exp(sc - sc.max())
                o = (w @ Vf[:s0 + t + 1, 0]) / w.sum()
                assert ulp_dist(out[a, t, hq], f16_rne_f64_array(o)).max() <= 1


ALL_PINS = [
    pin_bf16_rounding, pin_rope_hand_values, pin_rope_identity_at_zero, pin_rope_norm,
    pin_rope_vs_f64, pin_rope_relative, pin_single_key, pin_uniform_softmax, pin_constant_v,
    pin_dominant_key, pin_brute_force_f64, pin_gqa_equals_mha, pin_untouched_and_sentinel,
    pin_idempotent_and_permutation, pin_errors, pin_prefill_brute_force,
    pin_decode_after_prefill, pin_prefill_subset, pin_chunk_brute_force,
    pin_chunk_is_decode_steps, pin_ragged_groups, pin_chunk_errors, pin_f16_rounding,
    pin_f16_decode_brute_force, pin_f16_chunk_brute_force,
]
