"""CPU oracle for the positions-aware cached decode step and batched prefill.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this package.  It wraps the plain
C oracle (oracle/oracle.c) through ctypes; it shares no code with the HIP
library and imports nothing from it.

All arrays are numpy: BF16 tensors travel as uint16 bit patterns, indices as
int32.  The arithmetic, and the reading of every point the source pages leave
open, is documented in oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ERRORS = {1: "shape", 2: "index", 3: "duplicate row", 4: "out of memory"}


class OracleError(ValueError):
    pass


def _p(arr, ctype):
    return None if arr is None else arr.ctypes.data_as(ctypes.POINTER(ctype))


def _c(arr, dtype):
    return np.ascontiguousarray(arr, dtype=dtype)


def bf16_to_f32(bits):
    """BF16 bit patterns (uint16 array) -> float32 array (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# storage types of the 16-bit tensors (the oracle's ORC_BF16 / ORC_F16)
DTYPES = {"bf16": 1, "f16": 2}


class Oracle:
    """One loaded build of the oracle library (the default one, or a test mutant)."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIB
            if (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f32p = ctypes.POINTER(ctypes.c_float)
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_rope_inv_freq.argtypes = [ctypes.c_double, ctypes.c_int, f32p]
        L.orc_rope_cos_sin.argtypes = [ctypes.c_int, ctypes.c_int, f32p, f32p, f32p]
        L.orc_rope_apply.argtypes = [f32p, ctypes.c_int, f32p, f32p, f32p]
        L.orc_decode_step.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double] + [u16p] * 3 + \
            [i32p, i32p, u16p, u16p, u16p, f32p]
        L.orc_decode_step.restype = ctypes.c_int
        L.orc_prefill.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double] + [u16p] * 3 + \
            [i32p, u16p, u16p, u16p, i32p, ctypes.c_int]
        L.orc_prefill.restype = ctypes.c_int
        L.orc_prefill_chunk.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double] + [u16p] * 3 + \
            [i32p, i32p, i32p, u16p, u16p, u16p, i32p, ctypes.c_int]
        L.orc_prefill_chunk.restype = ctypes.c_int
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_decode_step_dt.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double] + [u16p] * 3 + \
            [i32p, i32p, u16p, u16p, u16p, f32p]
        L.orc_decode_step_dt.restype = ctypes.c_int
        L.orc_prefill_chunk_dt.argtypes = [ctypes.c_int] * 8 + [ctypes.c_double] + [u16p] * 3 + \
            [i32p, i32p, i32p, u16p, u16p, u16p, i32p, ctypes.c_int]
        L.orc_prefill_chunk_dt.restype = ctypes.c_int
        self.L = L
        self.path = path

    # -- scalar helpers ---------------------------------------------------------
    def f32_to_bf16(self, x):
        """float32 scalar -> BF16 bits, through the oracle's own rounding."""
        return int(self.L.orc_f32_to_bf16(float(x)))

    def bf16_to_f32(self, h):
        return float(self.L.orc_bf16_to_f32(int(h)))

    def f32_to_f16(self, x):
        """float32 scalar -> FP16 bits, through the oracle's own rounding."""
        return int(self.L.orc_f32_to_f16(float(x)))

    def f16_to_f32(self, h):
        return float(self.L.orc_f16_to_f32(int(h)))

    # -- RoPE -------------------------------------------------------------------
    def rope_inv_freq(self, base, D):
        out = np.zeros(D // 2, dtype=np.float32)
        self.L.orc_rope_inv_freq(float(base), int(D), _p(out, ctypes.c_float))
        return out

    def rope_cos_sin(self, pos, D, base):
        inv = self.rope_inv_freq(base, D)
        c = np.zeros(D // 2, dtype=np.float32)
        s = np.zeros(D // 2, dtype=np.float32)
        self.L.orc_rope_cos_sin(int(pos), int(D), _p(inv, ctypes.c_float),
                                _p(c, ctypes.c_float), _p(s, ctypes.c_float))
        return c, s

    def rope_apply(self, x, pos, base):
        """Rotate one FP32 head vector x[D] at position pos (FP32 result, unrounded)."""
        x = _c(x, np.float32)
        D = x.shape[0]
        c, s = self.rope_cos_sin(pos, D, base)
        y = np.zeros(D, dtype=np.float32)
        self.L.orc_rope_apply(_p(x, ctypes.c_float), D, _p(c, ctypes.c_float),
                              _p(s, ctypes.c_float), _p(y, ctypes.c_float))
        return y

    # -- the path ---------------------------------------------------------------
    def decode_step(self, q, k_new, v_new, positions, rows, Kc, Vc, base, want_f32=False,
                    dtype="bf16"):
        """One decode step.  Kc and Vc ([S, C, Hkv, D] uint16) are updated IN PLACE.
        dtype: "bf16" or "f16", the storage type the uint16 bit patterns hold.

        Returns out [A, Hq, D] uint16 (and the FP32 output before rounding if
        want_f32).  Raises OracleError on invalid arguments (nothing written).
        """
        q = _c(q, np.uint16)
        k_new = _c(k_new, np.uint16)
        v_new = _c(v_new, np.uint16)
        positions = _c(positions, np.int32)
        rows = _c(rows, np.int32)
        assert Kc.dtype == np.uint16 and Vc.dtype == np.uint16
        assert Kc.flags.c_contiguous and Vc.flags.c_contiguous
        A, Hq, D = q.shape
        S, C, Hkv, D2 = Kc.shape
        assert D2 == D and Vc.shape == Kc.shape
        assert k_new.shape == (A, Hkv, D) and v_new.shape == (A, Hkv, D)
        assert positions.shape == (A,) and rows.shape == (A,)
        out = np.zeros((A, Hq, D), dtype=np.uint16)
        of = np.zeros((A, Hq, D), dtype=np.float32) if want_f32 else None
        rc = self.L.orc_decode_step_dt(DTYPES[dtype], A, S, C, Hq, Hkv, D, float(base),
                                    _p(q, ctypes.c_uint16),
                                    _p(k_new, ctypes.c_uint16), _p(v_new, ctypes.c_uint16),
                                    _p(positions, ctypes.c_int32), _p(rows, ctypes.c_int32),
                                    _p(Kc, ctypes.c_uint16), _p(Vc, ctypes.c_uint16),
                                    _p(out, ctypes.c_uint16), _p(of, ctypes.c_float))
        if rc:
            raise OracleError(ERRORS.get(rc, str(rc)))
        return (out, of) if want_f32 else out

    def prefill(self, q, k_new, v_new, rows, Kc, Vc, base, t_list=None, starts=None, lens=None,
                out=None, dtype="bf16"):
        """Equal-length prefill, or a chunk appended at per-entry starts.
        q [A,T,Hq,D], k_new/v_new [A,T,Hkv,D] (uint16); starts [A] (None = 0);
        lens [A] (None = T): entry a uses its first lens[a] tokens only.

        Kc/Vc updated IN PLACE (slots start .. start+len-1 of each row).
        Returns out [A,T,Hq,D] uint16 (a fresh zero array, or `out` updated in
        place); with t_list only those query positions are computed, and rows
        t >= lens[a] are never written.
        """
        q = _c(q, np.uint16)
        k_new = _c(k_new, np.uint16)
        v_new = _c(v_new, np.uint16)
        rows = _c(rows, np.int32)
        assert Kc.flags.c_contiguous and Vc.flags.c_contiguous
        A, T, Hq, D = q.shape
        S, C, Hkv, _ = Kc.shape
        if out is None:
            out = np.zeros((A, T, Hq, D), dtype=np.uint16)
        assert out.dtype == np.uint16 and out.shape == (A, T, Hq, D) and out.flags.c_contiguous
        tl = None if t_list is None else _c(t_list, np.int32)
        st = None if starts is None else _c(starts, np.int32)
        ln = None if lens is None else _c(lens, np.int32)
        rc = self.L.orc_prefill_chunk_dt(DTYPES[dtype], A, T, S, C, Hq, Hkv, D, float(base),
                                _p(q, ctypes.c_uint16),
                                _p(k_new, ctypes.c_uint16), _p(v_new, ctypes.c_uint16),
                                _p(st, ctypes.c_int32), _p(ln, ctypes.c_int32),
                                _p(rows, ctypes.c_int32), _p(Kc, ctypes.c_uint16),
                                _p(Vc, ctypes.c_uint16), _p(out, ctypes.c_uint16),
                                _p(tl, ctypes.c_int32), 0 if tl is None else int(tl.shape[0]))
        if rc:
            raise OracleError(ERRORS.get(rc, str(rc)))
        return out


_default = None


def default():
    """The oracle built from oracle/oracle.c (built on first use if missing or stale)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode_step(*args, **kwargs):
    return default().decode_step(*args, **kwargs)


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def rope_apply(*args, **kwargs):
    return default().rope_apply(*args, **kwargs)
