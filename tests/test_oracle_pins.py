"""CPU tests: the oracle against its pins, and planted mistakes against the pins.

The mutants are textual edits of oracle/oracle.c compiled into a temporary
library: a flipped rotation sign, a wrong RoPE frequency exponent, cycled
instead of repeated GQA heads, a missing score scale, an exclusive causal
bound, truncating BF16 rounding, a store into the wrong row, an unrotated
query, a mirrored V store, a prefill chunk rotated, stored or attended as if
it began at position 0, FP16 conversions that truncate, round ties away,
misplace the subnormal quantum or the overflow threshold, or read and store
FP16 tensors as BF16.  Each must fail at least one pin.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


# (name, old text, new text, which occurrence (0-based) to replace)
MUTANTS = [
    ("rotation_sign", "y[i] = ac - bs;", "y[i] = ac + bs;", 0),
    ("rotation_sign_hi", "y[i + h] = bc + as;", "y[i + h] = bc - as;", 0),
    ("freq_exponent", "-2.0 * (double)i / (double)D", "-1.0 * (double)i / (double)D", 0),
    ("gqa_cycled", "int kv = hq / G;", "int kv = hq % Hkv;", 0),
    ("no_scale", "float sj = dot * scale;", "float sj = dot;", 0),
    ("exclusive_causal", "slot, pos[a], scale", "slot, pos[a] - 1 < 0 ? 0 : pos[a] - 1, scale", 0),
    ("truncating_bf16", "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))", "if (0)", 0),
    ("store_wrong_row", "uint16_t *kd = Kc + rows[a] * row", "uint16_t *kd = Kc + (long)a * row", 0),
    ("query_unrotated", "orc_rope_apply(x, D, cs, sn, y);\n            const uint16_t *Kr",
     "memcpy(y, x, sizeof(float) * (size_t)D);\n            const uint16_t *Kr", 0),
    ("v_mirrored", "vd[d] = v[d];", "vd[d] = v[D - 1 - d];", 0),
    ("angle_in_double", "float theta = p * inv_freq[i];",
     "double theta = (double)pos * pow(10000.0, 0.0) * (double)inv_freq[i] * (1.0 + 1e-6);", 0),
    ("prefill_position_offset", "orc_rope_cos_sin(s0 + t, D, inv_freq, cs, sn);\n            for (int h",
     "orc_rope_cos_sin(s0 + t + 1, D, inv_freq, cs, sn);\n            for (int h", 0),
    ("chunk_key_rotated_from_zero", "orc_rope_cos_sin(s0 + t, D, inv_freq, cs, sn);\n            for (int h",
     "orc_rope_cos_sin(t, D, inv_freq, cs, sn);\n            for (int h", 0),
    ("chunk_query_rotated_from_zero", "orc_rope_cos_sin(s0 + t, D, inv_freq, cs, sn);\n            for (int hq",
     "orc_rope_cos_sin(t, D, inv_freq, cs, sn);\n            for (int hq", 0),
    ("chunk_keys_from_chunk_only", "attend_one(dt, y, D, Kr, Vr, slot, s0 + t,",
     "attend_one(dt, y, D, Kr, Vr, slot, t,", 0),
    ("ragged_store_whole_chunk", "for (int t = 0; t < n; ++t) {\n            orc_rope_cos_sin",
     "for (int t = 0; t < T; ++t) {\n            orc_rope_cos_sin", 0),
    ("ragged_query_whole_chunk", "if (t >= n)\n                continue;", "", 0),
    ("f16_truncating", "if (fr > 0.5 || (fr == 0.5 && fmod(r, 2.0) == 1.0))", "if (0)", 0),
    ("f16_ties_away", "(fr == 0.5 && fmod(r, 2.0) == 1.0)", "(fr == 0.5)", 0),
    ("f16_subnormal_quantum", "if (ex < -14)\n        ex = -14;", "if (ex < -15)\n        ex = -15;", 0),
    ("f16_overflow_early", "if (x >= 65520.0)", "if (x >= 65504.0)", 0),
    ("f16_widen_bias", "ldexp((double)(1024 + fr), ex - 25)", "ldexp((double)(1024 + fr), ex - 24)", 0),
    ("f16_read_as_bf16", "return dt == ORC_F16 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h);",
     "return orc_bf16_to_f32(h);", 0),
    ("f16_store_as_bf16", "return dt == ORC_F16 ? orc_f32_to_f16(f) : orc_f32_to_bf16(f);",
     "return orc_f32_to_bf16(f);", 0),
    ("chunk_k_stored_from_zero", "uint16_t *kd = Kc + rows[a] * row + (long)(s0 + t) * slot",
     "uint16_t *kd = Kc + rows[a] * row + (long)t * slot", 0),
]


def _replace_nth(text, old, new, n):
    idx = -1
    for _ in range(n + 1):
        idx = text.find(old, idx + 1)
        assert idx >= 0, f"mutation anchor not found: {old!r}"
    return text[:idx] + new + text[idx + len(old):]


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mut):
    name, old, new, n = mut
    src = open(obuild.SRC).read()
    bad = _replace_nth(src, old, new, n)
    path = os.path.join(tmp_path, f"oracle_{name}.c")
    with open(path, "w") as f:
        f.write(bad)
    so = obuild.build(path, os.path.join(tmp_path, f"liboracle_{name}.so"))
    m = oracle.Oracle(so)
    failed = []
    for pin in PINS:
        try:
            pin(m)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
