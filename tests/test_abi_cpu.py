"""CPU tests of the C ABI: the library loads, exports every symbol declared in
include/mllm.h, and rejects every invalid argument before its first HIP call
(fake device pointers are safe here: no check reaches the device)."""
import ctypes
import os
import re

import pytest
import torch

import positions_aware_cached_amd as pac

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mllm.h")

FAKE = 0x7F0000000000  # 256-aligned fake device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mllm_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = pac.load()
    names = declared_functions()
    assert "mllm_decode_rope_store_attn" in names and "mllm_prefill_rope_store_attn" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pac.EXPORTS)


def test_abi_version():
    assert pac.load().mllm_abi_version() == 1


def test_cache_bytes_formula():
    # L * 2 * S * C * Hkv * D * 2 bytes
    assert pac.cache_bytes(1, 64, 4096, 8, 128) == 1 * 2 * 64 * 4096 * 8 * 128 * 2
    assert pac.cache_bytes(32, 256, 8192, 8, 128) == 32 * 2 * 256 * 8192 * 8 * 128 * 2
    for bad in [(0, 1, 1, 1, 64), (1, 0, 1, 1, 64), (1, 1, 0, 1, 64), (1, 1, 1, 0, 64)]:
        with pytest.raises(pac.MllmError) as e:
            pac.cache_bytes(*bad)
        assert e.value.name == "INVALID_ARG"
    with pytest.raises(pac.MllmError) as e:
        pac.cache_bytes(1, 1, 1, 1, 96)
    assert e.value.name == "UNSUPPORTED"


def fake_view(shape, addr=FAKE, strides=None, dtype=pac.BF16, device=0, nbytes=None):
    v = pac.TensorView()
    v.data = addr
    v.ndim = len(shape)
    v.dtype = dtype
    v.device = device
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    n = 1
    for s in shape:
        n *= s
    v.bytes = nbytes if nbytes is not None else n * 2
    for i, (s, st) in enumerate(zip(shape, strides)):
        v.shape[i] = s
        v.stride[i] = st
    return v


class FakeCache:
    """A cache wrapping fake device addresses (wrap makes no HIP call)."""

    def __init__(self, L=2, S=8, C=256, Hkv=2, D=64, dtype=pac.BF16):
        self.S, self.C, self.Hkv, self.D = S, C, Hkv, D
        lb = S * C * Hkv * D * 2
        self.k = [FAKE + 0x100000000 * (2 * l + 1) for l in range(L)]
        self.v = [FAKE + 0x100000000 * (2 * l + 2) for l in range(L)]
        d = pac.CacheDesc(L, S, C, Hkv, D, dtype, 0)
        ks = (ctypes.c_void_p * L)(*self.k)
        vs = (ctypes.c_void_p * L)(*self.v)
        h = ctypes.c_void_p()
        st = pac.load().mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h))
        assert st == 0, pac.last_error()
        self.cache = pac.Cache(h, d)
        self.lb = lb


def call_decode(fc, A=4, Hq=4, q=None, k=None, v=None, out=None, pos=FAKE + 0x10000,
                rows=FAKE + 0x20000, mirror=None, base=1e4, rotary=None, ws=FAKE + 0x40000000,
                ws_bytes=1 << 30, layer=0, opts=None, status=None):
    D = fc.D
    q = q or fake_view([A, Hq, D], FAKE + 0x1000000)
    k = k or fake_view([A, fc.Hkv, D], FAKE + 0x2000000)
    v = v or fake_view([A, fc.Hkv, D], FAKE + 0x3000000)
    out = out or fake_view([A, Hq, D], FAKE + 0x4000000)
    rope = pac.RopeDesc(base, D if rotary is None else rotary, 0)
    hm = None
    if mirror is not None:
        hm = (ctypes.c_int32 * len(mirror))(*mirror)
    o = opts or pac.DecodeOpts()
    return pac.load().mllm_decode_rope_store_attn(
        fc.cache.handle, layer, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(pos), ctypes.c_void_p(rows), A, hm, ctypes.byref(rope),
        ctypes.byref(out), ctypes.c_void_p(ws), ws_bytes, ctypes.c_void_p(status),
        ctypes.byref(o), None)


def expect(st, name):
    assert pac.STATUS[st] == name, (pac.STATUS[st], pac.last_error())
    assert pac.last_error()


def test_decode_rejections_before_device():
    fc = FakeCache()
    D = fc.D
    expect(call_decode(fc, layer=2), "INVALID_ARG")
    expect(call_decode(fc, A=-1), "INVALID_ARG")
    expect(call_decode(fc, Hq=3, q=fake_view([4, 3, D], FAKE + 0x1000000),
                       out=fake_view([4, 3, D], FAKE + 0x4000000)), "INVALID_ARG")
    expect(call_decode(fc, Hq=34, q=fake_view([4, 34, D], FAKE + 0x1000000),
                       out=fake_view([4, 34, D], FAKE + 0x4000000)), "UNSUPPORTED")  # G = 17
    expect(call_decode(fc, base=0.0), "INVALID_ARG")
    expect(call_decode(fc, base=float("inf")), "INVALID_ARG")
    expect(call_decode(fc, rotary=32), "UNSUPPORTED")
    # views
    expect(call_decode(fc, q=fake_view([4, 4, D], dtype=7)), "UNSUPPORTED")
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, device=1)), "INVALID_ARG")
    expect(call_decode(fc, k=fake_view([4, 1, D], FAKE + 0x2000000)), "INVALID_ARG")
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, strides=[4 * D, D, 2])),
           "UNSUPPORTED")   # D not contiguous
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, strides=[4 * D, 4, 1])),
           "UNSUPPORTED")   # head stride not a multiple of 8
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, strides=[-4 * D, D, 1])),
           "INVALID_ARG")   # negative stride
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000002)), "UNSUPPORTED")  # misaligned
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, nbytes=4 * 4 * D * 2 - 2)),
           "INVALID_ARG")   # view exceeds its storage
    expect(call_decode(fc, q=fake_view([4, 4, D], 0)), "INVALID_ARG")                 # null data
    # spans that overflow a 64-bit element offset (a product, then a sum) or run
    # past the end of the address space fail whatever bytes the view claims
    s59 = (1 << 61) + (1 << 59)   # 3 * s59 fits, 6 * s59 does not
    for strides in ([1 << 62, D, 1], [s59, s59, 1]):
        expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, strides=strides,
                                           nbytes=(1 << 64) - 1)), "INVALID_ARG")
    expect(call_decode(fc, q=fake_view([4, 4, D], (1 << 64) - 1024)), "INVALID_ARG")
    expect(call_decode(fc, pos=0), "INVALID_ARG")
    # workspace
    expect(call_decode(fc, ws=0), "WORKSPACE")
    expect(call_decode(fc, ws=FAKE + 0x40000010), "WORKSPACE")
    expect(call_decode(fc, ws_bytes=16), "WORKSPACE")
    # options
    o = pac.DecodeOpts()
    o.waves = -1
    expect(call_decode(fc, opts=o), "INVALID_ARG")
    o.waves = pac.MAX_WAVES + 1
    expect(call_decode(fc, opts=o), "INVALID_ARG")
    o.waves, o.kernel = 0, 5
    expect(call_decode(fc, opts=o), "INVALID_ARG")


def test_decode_alias_rejections():
    fc = FakeCache()
    D = fc.D
    # out overlapping q
    expect(call_decode(fc, out=fake_view([4, 4, D], FAKE + 0x1000000 + 256)), "ALIAS")
    # out inside the cache K block of the layer
    expect(call_decode(fc, out=fake_view([4, 4, D], fc.k[0] + 4096)), "ALIAS")
    # workspace overlapping the V block
    expect(call_decode(fc, ws=fc.v[0] + 0x100), "ALIAS")
    # status word inside the output
    expect(call_decode(fc, status=FAKE + 0x4000000 + 8), "ALIAS")
    # read-only inputs may overlap each other (k_new and v_new the same memory)
    st = call_decode(fc, mirror=[1, 2, 3, 300, 0, 1, 2, 3],
                     v=fake_view([4, fc.Hkv, D], FAKE + 0x2000000))
    expect(st, "OUT_OF_RANGE")  # got past the alias check to the mirror check


def test_decode_host_mirror_rejections():
    fc = FakeCache()
    expect(call_decode(fc, mirror=[1, 2, 3, 256, 0, 1, 2, 3]), "OUT_OF_RANGE")   # pos >= C
    expect(call_decode(fc, mirror=[1, 2, 3, -1, 0, 1, 2, 3]), "OUT_OF_RANGE")
    expect(call_decode(fc, mirror=[1, 2, 3, 4, 0, 1, 2, 8]), "OUT_OF_RANGE")     # row >= S
    expect(call_decode(fc, mirror=[1, 2, 3, 4, 0, 1, 2, 2]), "INVALID_ARG")      # duplicate row


def test_decode_zero_entries_is_noop():
    fc = FakeCache()
    st = call_decode(fc, A=0, ws=0, ws_bytes=0)
    assert st == 0, pac.last_error()


def test_workspace_size_and_rows():
    fc = FakeCache()
    # one size for every position; the default covers any wave count
    a = pac.decode_workspace_size(fc.cache, 4, 4, -1, waves=64)
    b = pac.decode_workspace_size(fc.cache, 4, 4, 10, waves=64)
    full = pac.decode_workspace_size(fc.cache, 4, 4, -1)
    assert a == b > 0 and full > a
    G, D = 4 // fc.Hkv, fc.D
    # one partial per (segment, head) and per wave of the launch, G heads each
    assert full >= 4 * 4 * D * 4 + (4 * fc.Hkv + pac.MAX_WAVES) * G * (D + 2) * 4
    with pytest.raises(pac.MllmError):
        pac.decode_workspace_size(fc.cache, 4, 3, -1)
    with pytest.raises(pac.MllmError):
        pac.decode_workspace_size(fc.cache, 4, 4, fc.C)
    assert fc.cache.row_length(3) == 0
    fc.cache.reset_row(3)
    with pytest.raises(pac.MllmError) as e:
        fc.cache.reset_row(fc.S)
    assert e.value.name == "OUT_OF_RANGE"
    k, v = fc.cache.layer_ptrs(1)
    assert (k, v) == (fc.k[1], fc.v[1])
    with pytest.raises(pac.MllmError):
        fc.cache.layer_ptrs(2)


def test_wrap_rejections():
    d = pac.CacheDesc(1, 2, 16, 1, 64, pac.BF16, 0)
    h = ctypes.c_void_p()
    L = pac.load()
    ks = (ctypes.c_void_p * 1)(FAKE)
    vs = (ctypes.c_void_p * 1)(FAKE + 64)     # overlaps K block
    expect(L.mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)), "ALIAS")
    vs = (ctypes.c_void_p * 1)(FAKE + 0x100008)
    expect(L.mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)), "UNSUPPORTED")
    vs = (ctypes.c_void_p * 1)(0)
    expect(L.mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)), "INVALID_ARG")
    vs = (ctypes.c_void_p * 1)((1 << 64) - 1024)  # the block would wrap past the top
    expect(L.mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)), "INVALID_ARG")
    assert "wraps" in pac.last_error()


def call_prefill(fc, A=2, T=16, Hq=4, rows_host=(0, 1), ws=FAKE + 0x40000000, ws_bytes=1 << 30,
                 q=None, out=None, opts=None):
    D = fc.D
    q = q or fake_view([A, T, Hq, D], FAKE + 0x1000000)
    k = fake_view([A, T, fc.Hkv, D], FAKE + 0x2000000)
    v = fake_view([A, T, fc.Hkv, D], FAKE + 0x3000000)
    out = out or fake_view([A, T, Hq, D], FAKE + 0x4000000)
    rope = pac.RopeDesc(1e4, D, 0)
    rh = (ctypes.c_int32 * max(1, len(rows_host)))(*rows_host)
    return pac.load().mllm_prefill_rope_store_attn(
        fc.cache.handle, 0, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(FAKE + 0x20000), rh, A, T, ctypes.byref(rope), ctypes.byref(out),
        ctypes.c_void_p(ws), ws_bytes, ctypes.byref(opts) if opts is not None else None, None)


def test_prefill_rejections_before_device():
    fc = FakeCache()
    expect(call_prefill(fc, T=0, q=fake_view([2, 0, 4, fc.D])), "INVALID_ARG")
    expect(call_prefill(fc, T=fc.C + 1), "INVALID_ARG")
    expect(call_prefill(fc, rows_host=(0, 0)), "INVALID_ARG")
    expect(call_prefill(fc, rows_host=(0, 9)), "OUT_OF_RANGE")
    expect(call_prefill(fc, ws=0), "WORKSPACE")
    expect(call_prefill(fc, out=fake_view([2, 16, 4, fc.D], FAKE + 0x1000000)), "ALIAS")


def call_chunk(fc, A=2, T=16, Hq=4, meta=(0, 5, 16, 16, 0, 1), meta_dev=FAKE + 0x20000,
               ws=FAKE + 0x40000000, ws_bytes=1 << 30, out=None):
    D = fc.D
    q = fake_view([A, T, Hq, D], FAKE + 0x1000000)
    k = fake_view([A, T, fc.Hkv, D], FAKE + 0x2000000)
    v = fake_view([A, T, fc.Hkv, D], FAKE + 0x3000000)
    out = out or fake_view([A, T, Hq, D], FAKE + 0x4000000)
    rope = pac.RopeDesc(1e4, D, 0)
    mh = None if meta is None else (ctypes.c_int32 * max(1, len(meta)))(*meta)
    return pac.load().mllm_prefill_chunk_rope_store_attn(
        fc.cache.handle, 0, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(meta_dev), mh, A, T, ctypes.byref(rope), ctypes.byref(out),
        ctypes.c_void_p(ws), ws_bytes, None, None)


def test_prefill_chunk_rejections_before_device():
    """meta = (starts[A], lengths[A], rows[A]); capacity 256, T = 16."""
    fc = FakeCache()
    expect(call_chunk(fc, meta=None), "INVALID_ARG")
    expect(call_chunk(fc, meta_dev=0), "INVALID_ARG")
    expect(call_chunk(fc, meta=(0, 5, 16, 16, 1, 1)), "INVALID_ARG")        # duplicate row
    expect(call_chunk(fc, meta=(0, 5, 16, 16, 0, 8)), "OUT_OF_RANGE")       # row past S
    expect(call_chunk(fc, meta=(0, 5, 16, 0, 0, 1)), "INVALID_ARG")         # length 0
    expect(call_chunk(fc, meta=(0, 5, 17, 16, 0, 1)), "INVALID_ARG")        # length > T
    expect(call_chunk(fc, meta=(-1, 5, 16, 16, 0, 1)), "OUT_OF_RANGE")      # negative start
    expect(call_chunk(fc, meta=(0, 241, 16, 16, 0, 1)), "OUT_OF_RANGE")     # past capacity
    expect(call_chunk(fc, meta=(0, 250, 16, 6, 0, 1), ws_bytes=8191), "WORKSPACE")
    expect(call_chunk(fc, ws=FAKE + 0x40000001), "WORKSPACE")
    expect(call_chunk(fc, meta_dev=FAKE + 0x4000000), "ALIAS")             # metadata in out
    assert call_chunk(fc, A=0, meta=None, meta_dev=0) == 0    # no entries: a no-op


def test_prefill_workspace_scales_with_entries():
    fc = FakeCache()
    for A, T in [(1, 16), (3, 16), (16, 256)]:
        want = A * T * (fc.D // 2) * 8
        assert pac.prefill_workspace_size(fc.cache, A, T, 4) == (want + 255) // 256 * 256


def test_dtype_rules():
    """One storage type per cache (BF16 or FP16); every view of a call carries
    the cache's type; unknown type codes are unsupported."""
    fc = FakeCache(dtype=pac.F16)
    D = fc.D
    f16 = lambda shape, addr: fake_view(shape, addr, dtype=pac.F16)
    q, k, v = f16([4, 4, D], FAKE + 0x1000000), f16([4, 2, D], FAKE + 0x2000000), \
        f16([4, 2, D], FAKE + 0x3000000)
    out = f16([4, 4, D], FAKE + 0x4000000)
    # FP16 views on an FP16 cache pass the checks (the call then fails only at
    # the device check: there is no GPU here)
    st = call_decode(fc, q=q, k=k, v=v, out=out, mirror=[1, 2, 3, 4, 0, 1, 2, 3])
    assert pac.STATUS[st] in ("DEVICE", "INVALID_ARG") and "dtype" not in pac.last_error()
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000), k=k, v=v, out=out),
           "INVALID_ARG")                                           # BF16 q on an FP16 cache
    expect(call_decode(fc, q=q, k=k, v=v, out=fake_view([4, 4, D], FAKE + 0x4000000)),
           "INVALID_ARG")                                           # BF16 out
    expect(call_decode(fc, q=fake_view([4, 4, D], FAKE + 0x1000000, dtype=3), k=k, v=v,
                       out=out), "UNSUPPORTED")
    d = pac.CacheDesc(1, 2, 16, 1, 64, 3, 0)
    h = ctypes.c_void_p()
    ks = (ctypes.c_void_p * 1)(FAKE)
    vs = (ctypes.c_void_p * 1)(FAKE + 0x100000)
    expect(pac.load().mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)), "UNSUPPORTED")
    assert pac.cache_bytes(1, 2, 16, 1, 64, dtype=pac.torch.float16) == \
        pac.cache_bytes(1, 2, 16, 1, 64)


def test_grid_size_limits():
    """One-dimensional launch grids count their work-items in 32 bits: the host
    refuses a call whose grid would not fit, before any launch (the decode
    merge: one 64-lane wave per entry and query head, so A * H_q < 2^26; the
    readable prefill: A * T * H_q < 2^26; the matrix-core prefill: A * H_q *
    ceil(T / 128) 256-lane blocks < 2^24)."""
    fc = FakeCache(S=8, C=256)
    G = 1 << 30
    views = lambda A, Hq: dict(q=fake_view([A, Hq, fc.D], FAKE + 1 * G),
                               k=fake_view([A, fc.Hkv, fc.D], FAKE + 2 * G),
                               v=fake_view([A, fc.Hkv, fc.D], FAKE + 3 * G),
                               out=fake_view([A, Hq, fc.D], FAKE + 4 * G),
                               pos=FAKE + 5 * G, rows=FAKE + 6 * G, mirror=None)
    A = 1 << 24
    expect(call_decode(fc, A=A, Hq=4, **views(A, 4)), "UNSUPPORTED")          # 2^26 waves
    st = call_decode(fc, A=A - 1, Hq=4, **views(A - 1, 4))                     # just below
    assert pac.STATUS[st] != "UNSUPPORTED", pac.last_error()
    # readable prefill: 2 x 256 tokens x 2^17 heads = 2^26 waves; the matrix-core
    # kernel takes the same shape (2^19 blocks)
    Hq = 1 << 17
    ro = pac.DecodeOpts()
    ro.kernel = 1
    expect(call_prefill(fc, A=2, T=256, Hq=Hq, rows_host=(0, 1), opts=ro), "UNSUPPORTED")
    st = call_prefill(fc, A=2, T=256, Hq=Hq, rows_host=(0, 1))
    assert "grid" not in pac.last_error(), pac.last_error()
    big = 1 << 29
    expect(call_prefill(fc, A=2, T=256, Hq=big // 64 * 32, rows_host=(0, 1)), "UNSUPPORTED")


def test_host_arrays_checked_by_the_binding():
    """Host-side index arrays cross the ABI as raw host pointers that the library
    reads for a fixed count: the binding refuses device tensors and wrong counts."""
    t, p = pac._host_i32([1, 2, 3, 4], 4, "host_mirror")
    assert t.dtype == torch.int32 and [p[i] for i in range(4)] == [1, 2, 3, 4]
    with pytest.raises(ValueError, match="hold 4"):
        pac._host_i32([1, 2, 3], 4, "host_mirror")
    with pytest.raises(ValueError, match="host memory"):
        pac._host_i32(torch.empty(4, dtype=torch.int32, device="meta"), 4, "rows_host")


def call_decode_noalloc(fc, A=4, Hq=4, q=None, k=None, v=None, out=None, pos=FAKE + 0x10000,
                        rows=FAKE + 0x20000, layer=0, opts=None):
    D = fc.D
    q = q or fake_view([A, Hq, D], FAKE + 0x1000000)
    k = k or fake_view([A, fc.Hkv, D], FAKE + 0x2000000)
    v = v or fake_view([A, fc.Hkv, D], FAKE + 0x3000000)
    out = out or fake_view([A, Hq, D], FAKE + 0x4000000)
    rope = pac.RopeDesc(1e4, D, 0)
    o = opts or pac.DecodeOpts()
    return pac.load().mllm_decode_rope_store_attn_noalloc(
        fc.cache.handle, layer, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(pos), ctypes.c_void_p(rows), A, None, ctypes.byref(rope),
        ctypes.byref(out), None, ctypes.byref(o), None)


def test_decode_noalloc_checks_and_limit():
    """The allocation-free decode call makes the checks of the workspace call,
    and refuses a call whose partials need more than its 64 MiB scratch before
    any device query."""
    fc = FakeCache()
    expect(call_decode_noalloc(fc, layer=2), "INVALID_ARG")
    expect(call_decode_noalloc(fc, pos=0), "INVALID_ARG")
    expect(call_decode_noalloc(fc, out=fake_view([4, 4, fc.D], fc.k[0] + 4096)), "ALIAS")
    o = pac.DecodeOpts()
    o.kernel = 5
    expect(call_decode_noalloc(fc, opts=o), "INVALID_ARG")
    assert call_decode_noalloc(fc, A=0) == 0, pac.last_error()
    # 20000 entries x 64 query heads x 64 dims: the FP32 rotated queries alone
    # take 328 MB of scratch
    big = FakeCache(Hkv=8, S=20000, C=16)
    A, Hq, D = 20000, 64, big.D
    G = 1 << 30
    st = call_decode_noalloc(big, A=A, Hq=Hq, q=fake_view([A, Hq, D], FAKE + 1 * G),
                             k=fake_view([A, 8, D], FAKE + 2 * G),
                             v=fake_view([A, 8, D], FAKE + 3 * G),
                             out=fake_view([A, Hq, D], FAKE + 4 * G),
                             pos=FAKE + 5 * G, rows=FAKE + 6 * G)
    expect(st, "UNSUPPORTED")
    assert "scratch" in pac.last_error()


# Section titles of the pages that define the boundary's operations.
SECTIONS = ("Tensor ownership boundary", "Attention layout boundary", "Tensor N0 invariants",
            "Stable integration boundary", "Correctness-first workflow", "Public interfaces",
            "Acceptance rule")


def test_every_declaration_cites_its_section():
    """Each mllm_* declaration of include/mllm.h is preceded by a comment that
    names the page section defining it (the allocation-free call names instead
    the callers it is for)."""
    text = open(HEADER).read()
    token = re.compile(r"/\*.*?\*/|\b(?:mllm_status|int|const char \*)\s*(mllm_[a-z_]+)\s*\(",
                       re.S)
    last, seen = "", []
    for m in token.finditer(text):
        if m.group(0).startswith("/*"):
            last = " ".join(re.sub(r"^\s*\*", " ", l) for l in m.group(0).splitlines())
            last = " ".join(last.split())
            continue
        name = m.group(1)
        seen.append(name)
        ok = any(t in last for t in SECTIONS)
        if name.endswith("_noalloc"):
            ok = "cannot allocate" in last
        assert ok, f"{name}: no section cited in its comment: {last[:120]}"
    assert set(seen) == set(declared_functions())
