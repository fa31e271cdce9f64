"""Small BF16 helpers for tests (independent of both the oracle and the HIP path).

Expected values here are built from closed forms in float64 and rounded by a
round-half-even on the binary significand written from the definition of
BF16 (8 significant bits, the exponent range of binary32).
"""
import math
import struct

import numpy as np


def bf16_exact(x):
    """BF16 bits of a value that is exactly representable (asserts exactness)."""
    u = struct.unpack("<I", struct.pack("<f", float(x)))[0]
    assert u & 0xFFFF == 0, f"{x} is not exactly representable in BF16"
    return u >> 16


def bf16_rne_f64(x):
    """Round a float64 value to BF16 (nearest, ties to even), directly from float64."""
    if x != x:
        return 0x7FC0
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    m, e = math.frexp(abs(x))          # |x| = m * 2^e, m in [0.5, 1)
    if e - 1 < -126:                   # subnormal range of binary32 / BF16
        q = abs(x) / 2.0 ** -133       # units of the smallest BF16 subnormal
        r = math.floor(q)
        f = q - r
        if f > 0.5 or (f == 0.5 and r % 2 == 1):
            r += 1
        v = r * 2.0 ** -133
    else:
        q = m * 256.0
        r = math.floor(q)
        f = q - r
        if f > 0.5 or (f == 0.5 and r % 2 == 1):
            r += 1
        v = r / 256.0 * 2.0 ** e
    if v >= 2.0 ** 128:
        b = 0x7F80
    else:
        b = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    return b | (0x8000 if x < 0 else 0)


def bf16_rne_f64_array(a):
    a = np.asarray(a, dtype=np.float64)
    return np.array([bf16_rne_f64(v) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def to_f32(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def ordered(bits):
    """Map BF16 codes to integers whose order is the numeric order (+0 == -0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_dist(a, b):
    """|ord(a) - ord(b)| elementwise for BF16 codes."""
    return np.abs(ordered(a) - ordered(b))


def rope_f64(x, pos, base):
    """Split-half RoPE in float64 from the closed form (pairs (i, i + D/2))."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    i = np.arange(h, dtype=np.float64)
    theta = float(pos) * base ** (-2.0 * i / D)
    c, s = np.cos(theta), np.sin(theta)
    lo = x[..., :h] * c - x[..., h:] * s
    hi = x[..., h:] * c + x[..., :h] * s
    return np.concatenate([lo, hi], axis=-1)


# ---- FP16 (IEEE binary16) codes: numpy's float16 is the library reference

def f16_to_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f16_rne_f64_array(a):
    """Round float64 values to FP16 codes (numpy's correctly rounded conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def widen(bits, dtype):
    """16-bit codes of storage type dtype ("bf16" / "f16") -> float32."""
    return f16_to_f32(bits) if dtype == "f16" else to_f32(bits)


def round_f64(a, dtype):
    return f16_rne_f64_array(a) if dtype == "f16" else bf16_rne_f64_array(a)
