"""Python binding of libmllm, the positions-aware cached decode library for MI355X.

Argument marshalling only: every step of the decode and prefill paths runs in
the library's HIP kernels.  PyTorch supplies device memory and streams; each
tensor crosses the C ABI (include/mllm.h) as a non-owning view.  The binding
fails loudly when the library is missing or a call is rejected; there is no
fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmllm.so")

OK = 0
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALIAS", 4: "OUT_OF_RANGE",
          5: "ROW_BUSY", 6: "WORKSPACE", 7: "OUT_OF_MEMORY", 8: "DEVICE"}
BF16 = 1
F16 = 2
# torch dtype -> storage type code of the C ABI
DTYPE_CODES = {torch.bfloat16: BF16, torch.float16: F16}

EXPORTS = ("mllm_abi_version", "mllm_last_error", "mllm_cache_bytes", "mllm_cache_alloc",
           "mllm_cache_wrap", "mllm_cache_free", "mllm_cache_layer", "mllm_cache_get_desc",
           "mllm_cache_reset_row", "mllm_cache_row_length", "mllm_decode_workspace_size",
           "mllm_decode_rope_store_attn", "mllm_prefill_workspace_size",
           "mllm_prefill_rope_store_attn", "mllm_prefill_chunk_rope_store_attn",
           "mllm_cache_set_row_length", "mllm_sched_create", "mllm_sched_free",
           "mllm_sched_max_sequence_length", "mllm_sched_submit", "mllm_sched_stop",
           "mllm_sched_cancel", "mllm_sched_boundary", "mllm_sched_counts",
           "mllm_decode_rope_store_attn_noalloc")


class MllmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class TensorView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("bytes", ctypes.c_uint64), ("ndim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("device", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("shape", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("device", ctypes.c_int32)]


class RopeDesc(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("rotary_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


MAX_WAVES = 4096  # largest wave count a decode launch accepts


class SchedEntry(ctypes.Structure):
    _fields_ = [("request_id", ctypes.c_int64), ("row", ctypes.c_int32), ("value", ctypes.c_int32)]


END_REASONS = {1: "length", 2: "stop", 3: "cancel"}


class DecodeOpts(ctypes.Structure):
    _fields_ = [("waves", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("attn_events", ctypes.c_void_p), ("reserved", ctypes.c_int32 * 4)]


_lib = None


def load(path=LIB_PATH):
    """Load libmllm.so (built by positions_aware_cached_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python positions_aware_cached_amd/build.py`")
    L = ctypes.CDLL(path)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    P = ctypes.POINTER
    L.mllm_abi_version.restype = ctypes.c_int
    L.mllm_last_error.restype = ctypes.c_char_p
    for name in EXPORTS[2:]:
        getattr(L, name).restype = ctypes.c_int
    L.mllm_cache_bytes.argtypes = [P(CacheDesc), P(u64)]
    L.mllm_cache_alloc.argtypes = [P(CacheDesc), P(vp)]
    L.mllm_cache_wrap.argtypes = [P(CacheDesc), P(vp), P(vp), P(vp)]
    L.mllm_cache_free.argtypes = [vp]
    L.mllm_cache_layer.argtypes = [vp, i32, P(vp), P(vp)]
    L.mllm_cache_get_desc.argtypes = [vp, P(CacheDesc)]
    L.mllm_cache_reset_row.argtypes = [vp, i32]
    L.mllm_cache_row_length.argtypes = [vp, i32, P(i32)]
    L.mllm_cache_set_row_length.argtypes = [vp, i32, i32]
    L.mllm_sched_create.argtypes = [vp, i32, P(vp)]
    L.mllm_sched_free.argtypes = [vp]
    L.mllm_sched_max_sequence_length.argtypes = [vp, P(i32)]
    L.mllm_sched_submit.argtypes = [vp, ctypes.c_int64, i32, i32]
    L.mllm_sched_stop.argtypes = [vp, ctypes.c_int64]
    L.mllm_sched_cancel.argtypes = [vp, ctypes.c_int64]
    L.mllm_sched_boundary.argtypes = [vp, P(SchedEntry), i32, P(i32), P(SchedEntry), i32, P(i32),
                                      P(SchedEntry), i32, P(i32)]
    L.mllm_sched_counts.argtypes = [vp, P(i32), P(i32)]
    L.mllm_decode_workspace_size.argtypes = [vp, i32, i32, i32, P(DecodeOpts), P(u64)]
    L.mllm_decode_rope_store_attn.argtypes = [
        vp, i32, P(TensorView), P(TensorView), P(TensorView), vp, vp, i32, P(i32),
        P(RopeDesc), P(TensorView), vp, u64, vp, P(DecodeOpts), vp]
    L.mllm_decode_rope_store_attn_noalloc.argtypes = [
        vp, i32, P(TensorView), P(TensorView), P(TensorView), vp, vp, i32, P(i32),
        P(RopeDesc), P(TensorView), vp, P(DecodeOpts), vp]
    L.mllm_prefill_workspace_size.argtypes = [vp, i32, i32, i32, P(u64)]
    L.mllm_prefill_rope_store_attn.argtypes = [
        vp, i32, P(TensorView), P(TensorView), P(TensorView), vp, P(i32), i32, i32,
        P(RopeDesc), P(TensorView), vp, u64, P(DecodeOpts), vp]
    L.mllm_prefill_chunk_rope_store_attn.argtypes = [
        vp, i32, P(TensorView), P(TensorView), P(TensorView), vp, P(i32), i32, i32,
        P(RopeDesc), P(TensorView), vp, u64, P(DecodeOpts), vp]
    _lib = L
    return L


def last_error():
    return load().mllm_last_error().decode()


def _check(status):
    if status != OK:
        raise MllmError(status, last_error())


def view(t):
    """Non-owning view of a torch tensor (pointer, accessible bytes, shape, strides)."""
    v = TensorView()
    if t is None:
        return None
    if t.dtype not in DTYPE_CODES:
        raise TypeError(f"expected a bfloat16 or float16 tensor, got {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    v.data = t.data_ptr() if t.numel() else (t.data_ptr() or None)
    v.bytes = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    v.ndim = t.dim()
    v.dtype = DTYPE_CODES[t.dtype]
    v.device = t.device.index if t.is_cuda else -1
    for i in range(t.dim()):
        v.shape[i] = t.shape[i]
        v.stride[i] = t.stride(i)
    return v


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _host_i32(x, n, name):
    """A host int32 copy of exactly n values (the library reads n values through
    the pointer, on the host): a tensor on a GPU or a wrong count is refused."""
    if isinstance(x, torch.Tensor) and x.device.type != "cpu":
        raise ValueError(f"{name} must be host memory, got a tensor on {x.device}")
    t = torch.as_tensor(x, dtype=torch.int32).contiguous().reshape(-1)
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} int32 values, got {t.numel()}")
    return t, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _opts(waves=0, kernel=0, attn_events=None):
    o = DecodeOpts()
    o.waves = waves
    o.kernel = kernel
    if attn_events is not None:
        o.attn_events = ctypes.cast(attn_events, ctypes.c_void_p)
    return o


def cache_bytes(num_layers, slots, capacity, h_kv, head_dim, device=0, dtype=torch.bfloat16):
    d = CacheDesc(num_layers, slots, capacity, h_kv, head_dim, DTYPE_CODES[dtype], device)
    n = ctypes.c_uint64()
    _check(load().mllm_cache_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


class Cache:
    """A shared slot cache: engine-owned (alloc) or wrapping torch tensors (wrap)."""

    def __init__(self, handle, desc, keep=None):
        self.handle = handle
        self.desc = desc
        self._keep = keep  # torch tensors that own wrapped memory

    @classmethod
    def alloc(cls, num_layers, slots, capacity, h_kv, head_dim, device=0, dtype=torch.bfloat16):
        d = CacheDesc(num_layers, slots, capacity, h_kv, head_dim, DTYPE_CODES[dtype], device)
        h = ctypes.c_void_p()
        _check(load().mllm_cache_alloc(ctypes.byref(d), ctypes.byref(h)))
        return cls(h, d)

    @classmethod
    def wrap(cls, k_layers, v_layers):
        """Wrap lists of [slots, capacity, h_kv, head_dim] CUDA tensors (one per layer), all
        bfloat16 or all float16."""
        if len(k_layers) != len(v_layers) or not k_layers:
            raise ValueError("need the same positive number of K and V layers")
        t0 = k_layers[0]
        for t in list(k_layers) + list(v_layers):
            if (t.dtype != t0.dtype or t.dtype not in DTYPE_CODES or t.shape != t0.shape
                    or not t.is_contiguous()):
                raise ValueError("every layer block must be a contiguous tensor of one shape and "
                                 "one dtype (bfloat16 or float16)")
        S, C, Hkv, D = t0.shape
        dev = t0.device.index if t0.is_cuda else -1
        d = CacheDesc(len(k_layers), S, C, Hkv, D, DTYPE_CODES[t0.dtype], dev)
        n = len(k_layers)
        ks = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_layers])
        vs = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_layers])
        h = ctypes.c_void_p()
        _check(load().mllm_cache_wrap(ctypes.byref(d), ks, vs, ctypes.byref(h)))
        return cls(h, d, keep=(list(k_layers), list(v_layers)))

    def free(self):
        if self.handle:
            _check(load().mllm_cache_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def layer_ptrs(self, layer):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _check(load().mllm_cache_layer(self.handle, layer, ctypes.byref(k), ctypes.byref(v)))
        return k.value, v.value

    def reset_row(self, row):
        _check(load().mllm_cache_reset_row(self.handle, row))

    def row_length(self, row):
        n = ctypes.c_int32()
        _check(load().mllm_cache_row_length(self.handle, row, ctypes.byref(n)))
        return n.value

    def set_row_length(self, row, length):
        _check(load().mllm_cache_set_row_length(self.handle, row, length))


class Scheduler:
    """The slot manager over a cache (see mllm_sched_* in include/mllm.h)."""

    def __init__(self, cache, max_sequence_length=0):
        self.cache = cache  # kept alive: the scheduler reads and resets its rows
        self.slots = cache.desc.slots
        h = ctypes.c_void_p()
        _check(load().mllm_sched_create(cache.handle, max_sequence_length, ctypes.byref(h)))
        self.handle = h
        n = ctypes.c_int32()
        _check(load().mllm_sched_max_sequence_length(self.handle, ctypes.byref(n)))
        self.max_sequence_length = n.value
        # plan arrays and counts, reused by every boundary call
        self._arrs = [(SchedEntry * self.slots)() for _ in range(3)]
        self._ns = [ctypes.c_int32() for _ in range(3)]
        self._args = (self.handle, self._arrs[0], self.slots, ctypes.byref(self._ns[0]),
                      self._arrs[1], self.slots, ctypes.byref(self._ns[1]), self._arrs[2],
                      self.slots, ctypes.byref(self._ns[2]))

    def submit(self, request_id, prompt_len, max_new_tokens):
        _check(load().mllm_sched_submit(self.handle, request_id, prompt_len, max_new_tokens))

    def stop(self, request_id):
        _check(load().mllm_sched_stop(self.handle, request_id))

    def cancel(self, request_id):
        _check(load().mllm_sched_cancel(self.handle, request_id))

    def boundary(self):
        """One step boundary -> (admitted, decode, retired), each a list of
        (request_id, row, value) tuples (value: prompt length, position, end reason)."""
        self.boundary_native()
        return self.last_plan()

    def boundary_native(self):
        """The boundary call alone: the plan stays in the preallocated arrays
        (read it with last_plan())."""
        if not self.cache.handle:
            raise RuntimeError("the scheduler's cache has been freed")
        _check(load().mllm_sched_boundary(*self._args))

    def last_plan(self):
        """The plan of the last boundary call, as boundary() returns it."""
        return tuple([(e.request_id, e.row, e.value) for e in a[:n.value]]
                     for a, n in zip(self._arrs, self._ns))

    def counts(self):
        q, a = ctypes.c_int32(), ctypes.c_int32()
        _check(load().mllm_sched_counts(self.handle, ctypes.byref(q), ctypes.byref(a)))
        return q.value, a.value

    def free(self):
        if self.handle:
            _check(load().mllm_sched_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def decode_workspace_size(cache, A, h_q, max_position=-1, waves=0, kernel=0):
    n = ctypes.c_uint64()
    o = _opts(waves, kernel)
    _check(load().mllm_decode_workspace_size(cache.handle, A, h_q, max_position,
                                             ctypes.byref(o), ctypes.byref(n)))
    return n.value


def decode_rope_store_attn(cache, layer, q, k_new, v_new, positions, rows, out, workspace,
                           base, host_mirror=None, status=None, waves=0, kernel=0,
                           attn_events=None, stream=None):
    """One decode step of one layer (see mllm_decode_rope_store_attn in include/mllm.h).

    q [A,Hq,D], k_new/v_new [A,Hkv,D], out [A,Hq,D]: bf16 CUDA tensors.
    positions, rows: int32 CUDA tensors [A].  workspace: uint8 CUDA tensor.
    host_mirror: optional int32 CPU tensor/array of 2*A (positions then rows).
    attn_events: optional ctypes array of two hipEvent_t handles recorded around
    the attention kernel.
    """
    A = q.shape[0]
    rope = RopeDesc(float(base), q.shape[-1], 0)
    o = _opts(waves, kernel, attn_events)
    hm = None
    if host_mirror is not None:
        hm_t, hm = _host_i32(host_mirror, 2 * A, "host_mirror")
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().mllm_decode_rope_store_attn(
        cache.handle, layer, ctypes.byref(view(q)), ctypes.byref(view(k_new)),
        ctypes.byref(view(v_new)), _ptr(positions), _ptr(rows), A, hm, ctypes.byref(rope),
        ctypes.byref(view(out)), ws_ptr, ws_bytes, _ptr(status), ctypes.byref(o),
        _stream(stream)))


def decode_rope_store_attn_noalloc(cache, layer, q, k_new, v_new, positions, rows, out, base,
                                   host_mirror=None, status=None, waves=0, kernel=0,
                                   attn_events=None, stream=None):
    """The decode step without a workspace (mllm_decode_rope_store_attn_noalloc):
    the library's per-device scratch holds the partials; arguments as for
    decode_rope_store_attn."""
    A = q.shape[0]
    rope = RopeDesc(float(base), q.shape[-1], 0)
    o = _opts(waves, kernel, attn_events)
    hm = None
    if host_mirror is not None:
        hm_t, hm = _host_i32(host_mirror, 2 * A, "host_mirror")
    _check(load().mllm_decode_rope_store_attn_noalloc(
        cache.handle, layer, ctypes.byref(view(q)), ctypes.byref(view(k_new)),
        ctypes.byref(view(v_new)), _ptr(positions), _ptr(rows), A, hm, ctypes.byref(rope),
        ctypes.byref(view(out)), _ptr(status), ctypes.byref(o), _stream(stream)))


def prefill_workspace_size(cache, A, T, h_q):
    n = ctypes.c_uint64()
    _check(load().mllm_prefill_workspace_size(cache.handle, A, T, h_q, ctypes.byref(n)))
    return n.value


def prefill_rope_store_attn(cache, layer, q, k_new, v_new, rows_dev, rows_host, out, workspace,
                            base, kernel=0, attn_events=None, stream=None):
    """Equal-length prefill of one layer (see mllm_prefill_rope_store_attn).

    kernel: 0 matrix-core kernel, 1 readable kernel.
    """
    A, T = q.shape[0], q.shape[1]
    rope = RopeDesc(float(base), q.shape[-1], 0)
    o = _opts(0, kernel, attn_events)
    rh, rh_p = _host_i32(rows_host, A, "rows_host")
    _check(load().mllm_prefill_rope_store_attn(
        cache.handle, layer, ctypes.byref(view(q)), ctypes.byref(view(k_new)),
        ctypes.byref(view(v_new)), _ptr(rows_dev), rh_p, A, T, ctypes.byref(rope),
        ctypes.byref(view(out)), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        ctypes.byref(o), _stream(stream)))


def prefill_chunk_rope_store_attn(cache, layer, q, k_new, v_new, chunk_dev, chunk_host, out,
                                  workspace, base, kernel=0, attn_events=None, stream=None):
    """Prefill chunk at per-entry starts and lengths (see
    mllm_prefill_chunk_rope_store_attn).  chunk_dev: device int32 [3, A] or
    [3*A] = (starts, lengths, rows); chunk_host: the same values on the host.
    """
    A, T = q.shape[0], q.shape[1]
    rope = RopeDesc(float(base), q.shape[-1], 0)
    o = _opts(0, kernel, attn_events)
    ch, ch_p = _host_i32(chunk_host, 3 * A, "chunk_host")
    if chunk_dev is not None and chunk_dev.numel() != 3 * A:
        raise ValueError("chunk metadata must hold 3 * A int32 values")
    _check(load().mllm_prefill_chunk_rope_store_attn(
        cache.handle, layer, ctypes.byref(view(q)), ctypes.byref(view(k_new)),
        ctypes.byref(view(v_new)), _ptr(chunk_dev), ch_p, A, T, ctypes.byref(rope),
        ctypes.byref(view(out)), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        ctypes.byref(o), _stream(stream)))


class DecodeCall:
    """A decode call with every argument marshalled once (for tight loops).

    The tensors must stay alive and unchanged in shape while the object is
    used; `__call__(layer)` issues one decode step of that layer on `stream`.
    """

    def __init__(self, cache, q, k_new, v_new, positions, rows, out, workspace, base,
                 host_mirror=None, status=None, waves=0, kernel=0, stream=None):
        self.L = load()
        self.cache = cache
        self._keep = (q, k_new, v_new, positions, rows, out, workspace, status)
        self.A = q.shape[0]
        self.vq, self.vk, self.vv, self.vo = view(q), view(k_new), view(v_new), view(out)
        self.rope = RopeDesc(float(base), q.shape[-1], 0)
        self.opts = _opts(waves, kernel)
        self.hm_t = None
        self.hm = None
        if host_mirror is not None:
            self.hm_t, self.hm = _host_i32(host_mirror, 2 * self.A, "host_mirror")
        self.args_tail = (_ptr(positions), _ptr(rows), self.A, self.hm, ctypes.byref(self.rope),
                          ctypes.byref(self.vo), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _ptr(status))
        self.stream = _stream(stream)

    def __call__(self, layer, attn_events=None):
        self.opts.attn_events = (ctypes.cast(attn_events, ctypes.c_void_p).value
                                 if attn_events is not None else None)
        st = self.L.mllm_decode_rope_store_attn(
            self.cache.handle, layer, ctypes.byref(self.vq), ctypes.byref(self.vk),
            ctypes.byref(self.vv), *self.args_tail, ctypes.byref(self.opts), self.stream)
        if st != OK:
            raise MllmError(st, last_error())
