// mllm.cpp -- host layer of the C ABI declared in include/mllm.h.
//
// Argument checks, the cache object, workspace sizing and kernel dispatch.
// Every check runs before the first HIP call, so a rejected call has no side
// effect and the checks are testable on a machine without a GPU
// (microLLM-rocm ARCHITECTURE.md, "Tensor N0 invariants": negative dims and
// strides are rejected, zero-size dims are legal, a view must lie inside its
// storage, unsupported operations fail explicitly).
#include <hip/hip_runtime.h>
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mllm.h"
#include "host.h"
#include "kernels.h"

struct mllm_cache {
    mllm_cache_desc desc;
    bool owned;
    void *block;                 // owned allocation (all layers), or null
    std::vector<void *> k, v;    // per-layer block pointers
    std::vector<int32_t> length; // logical length of every row
};

namespace {

thread_local std::string g_error;

mllm_status fail(mllm_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

mllm_status ok()
{
    g_error.clear();
    return MLLM_OK;
}

}  // namespace

namespace mllm {

mllm_status host_fail(mllm_status st, const char *msg)
{
    return fail(st, "%s", msg);
}

mllm_status host_ok() { return ok(); }

}  // namespace mllm

namespace {

mllm_status hip_fail(hipError_t e, const char *what)
{
    return fail(MLLM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kElem = 2;  // bytes of a BF16 or FP16 element

mllm_status check_desc(const mllm_cache_desc *d)
{
    if (!d)
        return fail(MLLM_ERR_INVALID_ARG, "cache descriptor is null");
    if (d->num_layers <= 0 || d->slots <= 0 || d->capacity <= 0 || d->h_kv <= 0)
        return fail(MLLM_ERR_INVALID_ARG,
                    "num_layers, slots, capacity and h_kv must be positive (got %d %d %d %d)",
                    d->num_layers, d->slots, d->capacity, d->h_kv);
    if (d->dtype != MLLM_BF16 && d->dtype != MLLM_F16)
        return fail(MLLM_ERR_UNSUPPORTED, "cache dtype %d unsupported (BF16 or FP16)", d->dtype);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(MLLM_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
    if (d->device < 0)
        return fail(MLLM_ERR_INVALID_ARG, "device ordinal %d is negative", d->device);
    if ((uint64_t)d->capacity * d->h_kv * d->head_dim * 2 >= (1ull << 31))
        return fail(MLLM_ERR_UNSUPPORTED, "one cache row (capacity * h_kv * head_dim * 2 bytes) "
                    "must stay below 2 GiB");
    if (d->capacity >= (1 << 24))
        return fail(MLLM_ERR_UNSUPPORTED, "capacity must be below 2^24");
    return MLLM_OK;
}

uint64_t layer_bytes(const mllm_cache_desc &d)
{
    return (uint64_t)d.slots * (uint64_t)d.capacity * (uint64_t)d.h_kv * (uint64_t)d.head_dim *
           (uint64_t)kElem;
}

// A byte range used for the alias checks.
struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
    bool writable;
};

bool overlap(const Range &a, const Range &b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

mllm_status check_aliases(const std::vector<Range> &r)
{
    for (const Range &x : r)
        if (x.hi < x.lo)
            return fail(MLLM_ERR_INVALID_ARG, "%s wraps around the end of the address space",
                        x.name);
    for (size_t i = 0; i < r.size(); ++i)
        for (size_t j = i + 1; j < r.size(); ++j)
            if ((r[i].writable || r[j].writable) && overlap(r[i], r[j]))
                return fail(MLLM_ERR_ALIAS, "%s overlaps %s", r[i].name, r[j].name);
    return MLLM_OK;
}

// Validate a view against an expected shape and the cache's dtype and
// device; returns its byte range.
mllm_status check_view(const mllm_tensor_view *v, const char *name, int ndim,
                       const int64_t *shape, int device, int dtype, bool writable, Range *range)
{
    if (!v)
        return fail(MLLM_ERR_INVALID_ARG, "%s view is null", name);
    if (v->ndim != ndim)
        return fail(MLLM_ERR_INVALID_ARG, "%s must have %d dims (got %d)", name, ndim, v->ndim);
    if (v->dtype != MLLM_BF16 && v->dtype != MLLM_F16)
        return fail(MLLM_ERR_UNSUPPORTED, "%s dtype %d unsupported (BF16 or FP16)", name,
                    v->dtype);
    if (v->dtype != dtype)
        return fail(MLLM_ERR_INVALID_ARG, "%s dtype %d differs from the cache's %d", name,
                    v->dtype, dtype);
    if (v->device != device)
        return fail(MLLM_ERR_INVALID_ARG, "%s is on device %d, cache on %d", name, v->device,
                    device);
    int64_t numel = 1;
    for (int k = 0; k < ndim; ++k) {
        if (v->shape[k] < 0 || v->stride[k] < 0)
            return fail(MLLM_ERR_INVALID_ARG, "%s has a negative dim or stride", name);
        if (v->shape[k] != shape[k])
            return fail(MLLM_ERR_INVALID_ARG, "%s dim %d is %lld, expected %lld", name, k,
                        (long long)v->shape[k], (long long)shape[k]);
        numel *= v->shape[k];
    }
    if (v->stride[ndim - 1] != 1)
        return fail(MLLM_ERR_UNSUPPORTED, "%s: head dimension must be contiguous", name);
    for (int k = 0; k < ndim - 1; ++k)
        if (v->stride[k] % 8 != 0)
            return fail(MLLM_ERR_UNSUPPORTED, "%s: stride of dim %d must be a multiple of 8 "
                        "elements (16-byte rows)", name, k);
    if (numel == 0) {
        *range = Range{name, 0, 0, writable};
        return MLLM_OK;
    }
    if (!v->data)
        return fail(MLLM_ERR_INVALID_ARG, "%s data pointer is null", name);
    if (((uintptr_t)v->data) % 16 != 0)
        return fail(MLLM_ERR_UNSUPPORTED, "%s data must be 16-byte aligned", name);
    // element offset of the last element, and the bytes up to its end, with
    // every product and sum checked (strides are the caller's)
    int64_t last = 0;
    for (int k = 0; k < ndim; ++k) {
        int64_t term = 0;
        if (__builtin_mul_overflow(v->shape[k] - 1, v->stride[k], &term) ||
            __builtin_add_overflow(last, term, &last))
            return fail(MLLM_ERR_INVALID_ARG, "%s: its shape and strides span more elements "
                        "than a 64-bit offset holds", name);
    }
    uint64_t need = 0;
    if (__builtin_mul_overflow((uint64_t)last + 1u, (uint64_t)kElem, &need) ||
        (uintptr_t)v->data + need < (uintptr_t)v->data)
        return fail(MLLM_ERR_INVALID_ARG, "%s: its span runs past the end of the address space",
                    name);
    if (need > v->bytes)
        return fail(MLLM_ERR_INVALID_ARG, "%s spans %llu bytes but only %llu are accessible",
                    name, (unsigned long long)need, (unsigned long long)v->bytes);
    *range = Range{name, (uintptr_t)v->data, (uintptr_t)v->data + need, writable};
    return MLLM_OK;
}

mllm_status check_rope(const mllm_rope_desc *r, int D)
{
    if (!r)
        return fail(MLLM_ERR_INVALID_ARG, "rope descriptor is null");
    if (!(std::isfinite(r->base) && r->base > 0.0))
        return fail(MLLM_ERR_INVALID_ARG, "rope base must be finite and positive");
    if (r->rotary_dim != D)
        return fail(MLLM_ERR_UNSUPPORTED, "rotary_dim %d must equal head_dim %d", r->rotary_dim,
                    D);
    return MLLM_OK;
}

// inv_freq[i] = fl32(base^(-2i/D)), evaluated in double.
void fill_inv_freq(float *inv, double base, int D)
{
    for (int i = 0; i < D / 2; ++i)
        inv[i] = (float)std::pow(base, -2.0 * (double)i / (double)D);
}

mllm_status resolve_opts(const mllm_decode_opts *opts, int *waves, int *kernel)
{
    *waves = 0;
    *kernel = 0;
    if (!opts)
        return MLLM_OK;
    for (int i = 0; i < 4; ++i)
        if (opts->reserved[i] != 0)
            return fail(MLLM_ERR_INVALID_ARG, "reserved option fields must be zero");
    if (opts->waves < 0 || opts->waves > MLLM_MAX_WAVES)
        return fail(MLLM_ERR_INVALID_ARG, "waves %d must be 0 (device default) or in [1, %d]",
                    opts->waves, MLLM_MAX_WAVES);
    *waves = opts->waves;
    if (opts->kernel != 0 && opts->kernel != 1)
        return fail(MLLM_ERR_INVALID_ARG, "kernel %d unknown (0 tuned, 1 readable)",
                    opts->kernel);
    *kernel = opts->kernel;
    return MLLM_OK;
}

// Work groups of a decode launch (hg waves each, one per kv head of a head
// group): the waves option divided by hg, else the device's resident groups
// for the kernel variant (queried once per device and shape).
int launch_groups(int requested_waves, int device, int D, int G, int hg, int dtype)
{
    if (requested_waves > 0)
        return std::max(1, requested_waves / hg);
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int, int>, int> cache;
    const int gcls = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_tuple(device, D, gcls, hg, dtype);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int ng = mllm::decode_resident_groups(device, D, G, hg, dtype);
    if (ng <= 0)
        ng = 2048 / hg;
    ng = std::min(ng, MLLM_MAX_WAVES / hg);
    cache[key] = ng;
    return ng;
}

// Compute units of a device (queried once per device).
int device_cus(int device)
{
    static std::mutex mu;
    static std::map<int, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(device);
    if (it != cache.end())
        return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        cus = 0;
    cache[device] = cus;
    return cus;
}

// A one-dimensional launch of `blocks` work groups of `threads` work-items:
// the dispatch packet counts the grid's work-items in 32 bits.
bool grid_fits(int64_t blocks, int threads)
{
    return blocks >= 0 && blocks < (int64_t(1) << 32) / threads;
}

mllm_status check_device_current(int device)
{
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (cur != device)
        return fail(MLLM_ERR_INVALID_ARG, "current device is %d but the cache is on %d", cur,
                    device);
    return MLLM_OK;
}

}  // namespace

extern "C" {

int mllm_abi_version(void) { return MLLM_ABI_VERSION; }

const char *mllm_last_error(void) { return g_error.c_str(); }

mllm_status mllm_cache_bytes(const mllm_cache_desc *desc, uint64_t *bytes)
{
    mllm_status st = check_desc(desc);
    if (st)
        return st;
    if (!bytes)
        return fail(MLLM_ERR_INVALID_ARG, "bytes is null");
    *bytes = (uint64_t)desc->num_layers * 2u * layer_bytes(*desc);
    return ok();
}

mllm_status mllm_cache_alloc(const mllm_cache_desc *desc, mllm_cache **out)
{
    mllm_status st = check_desc(desc);
    if (st)
        return st;
    if (!out)
        return fail(MLLM_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    const uint64_t lb = layer_bytes(*desc);
    const uint64_t total = (uint64_t)desc->num_layers * 2u * lb;
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    e = hipSetDevice(desc->device);
    if (e != hipSuccess)
        return hip_fail(e, "hipSetDevice");
    void *block = nullptr;
    e = hipMalloc(&block, total);
    (void)hipSetDevice(prev);
    if (e != hipSuccess)
        return fail(MLLM_ERR_OUT_OF_MEMORY, "hipMalloc of %llu bytes: %s",
                    (unsigned long long)total, hipGetErrorString(e));
    mllm_cache *c = new mllm_cache();
    c->desc = *desc;
    c->owned = true;
    c->block = block;
    for (int l = 0; l < desc->num_layers; ++l) {
        c->k.push_back((char *)block + (uint64_t)(2 * l) * lb);
        c->v.push_back((char *)block + (uint64_t)(2 * l + 1) * lb);
    }
    c->length.assign(desc->slots, 0);
    *out = c;
    return ok();
}

mllm_status mllm_cache_wrap(const mllm_cache_desc *desc, void *const *k_layers,
                            void *const *v_layers, mllm_cache **out)
{
    mllm_status st = check_desc(desc);
    if (st)
        return st;
    if (!out || !k_layers || !v_layers)
        return fail(MLLM_ERR_INVALID_ARG, "out, k_layers and v_layers must be non-null");
    *out = nullptr;
    const uint64_t lb = layer_bytes(*desc);
    std::vector<Range> ranges;
    for (int l = 0; l < desc->num_layers; ++l) {
        if (!k_layers[l] || !v_layers[l])
            return fail(MLLM_ERR_INVALID_ARG, "layer %d pointer is null", l);
        if (((uintptr_t)k_layers[l]) % 16 || ((uintptr_t)v_layers[l]) % 16)
            return fail(MLLM_ERR_UNSUPPORTED, "layer %d blocks must be 16-byte aligned", l);
        ranges.push_back(Range{"cache K block", (uintptr_t)k_layers[l],
                               (uintptr_t)k_layers[l] + lb, true});
        ranges.push_back(Range{"cache V block", (uintptr_t)v_layers[l],
                               (uintptr_t)v_layers[l] + lb, true});
    }
    st = check_aliases(ranges);
    if (st)
        return st;
    mllm_cache *c = new mllm_cache();
    c->desc = *desc;
    c->owned = false;
    c->block = nullptr;
    c->k.assign(k_layers, k_layers + desc->num_layers);
    c->v.assign(v_layers, v_layers + desc->num_layers);
    c->length.assign(desc->slots, 0);
    *out = c;
    return ok();
}

mllm_status mllm_cache_free(mllm_cache *cache)
{
    if (!cache)
        return ok();
    mllm_status st = MLLM_OK;
    if (cache->owned && cache->block) {
        hipError_t e = hipFree(cache->block);
        if (e != hipSuccess)
            st = hip_fail(e, "hipFree");
    }
    delete cache;
    return st ? st : ok();
}

mllm_status mllm_cache_layer(const mllm_cache *cache, int32_t layer, void **k, void **v)
{
    if (!cache || !k || !v)
        return fail(MLLM_ERR_INVALID_ARG, "cache, k and v must be non-null");
    if (layer < 0 || layer >= cache->desc.num_layers)
        return fail(MLLM_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer,
                    cache->desc.num_layers);
    *k = cache->k[layer];
    *v = cache->v[layer];
    return ok();
}

mllm_status mllm_cache_get_desc(const mllm_cache *cache, mllm_cache_desc *desc)
{
    if (!cache || !desc)
        return fail(MLLM_ERR_INVALID_ARG, "cache and desc must be non-null");
    *desc = cache->desc;
    return ok();
}

mllm_status mllm_cache_reset_row(mllm_cache *cache, int32_t row)
{
    if (!cache)
        return fail(MLLM_ERR_INVALID_ARG, "cache is null");
    if (row < 0 || row >= cache->desc.slots)
        return fail(MLLM_ERR_OUT_OF_RANGE, "row %d out of range [0, %d)", row,
                    cache->desc.slots);
    cache->length[row] = 0;
    return ok();
}

mllm_status mllm_cache_set_row_length(mllm_cache *cache, int32_t row, int32_t len)
{
    if (!cache)
        return fail(MLLM_ERR_INVALID_ARG, "cache is null");
    if (row < 0 || row >= cache->desc.slots)
        return fail(MLLM_ERR_OUT_OF_RANGE, "row %d out of range [0, %d)", row,
                    cache->desc.slots);
    if (len < 0 || len > cache->desc.capacity)
        return fail(MLLM_ERR_OUT_OF_RANGE, "length %d outside [0, capacity %d]", len,
                    cache->desc.capacity);
    cache->length[row] = len;
    return ok();
}

mllm_status mllm_cache_row_length(const mllm_cache *cache, int32_t row, int32_t *len)
{
    if (!cache || !len)
        return fail(MLLM_ERR_INVALID_ARG, "cache and len must be non-null");
    if (row < 0 || row >= cache->desc.slots)
        return fail(MLLM_ERR_OUT_OF_RANGE, "row %d out of range [0, %d)", row,
                    cache->desc.slots);
    *len = cache->length[row];
    return ok();
}

mllm_status mllm_decode_workspace_size(const mllm_cache *cache, int32_t A, int32_t h_q,
                                       int32_t max_position, const mllm_decode_opts *opts,
                                       uint64_t *bytes)
{
    if (!cache || !bytes)
        return fail(MLLM_ERR_INVALID_ARG, "cache and bytes must be non-null");
    const mllm_cache_desc &d = cache->desc;
    if (A < 0)
        return fail(MLLM_ERR_INVALID_ARG, "A must be >= 0");
    if (h_q <= 0 || h_q % d.h_kv != 0)
        return fail(MLLM_ERR_INVALID_ARG, "h_q %d must be a positive multiple of h_kv %d", h_q,
                    d.h_kv);
    if (max_position < -1 || max_position >= d.capacity)
        return fail(MLLM_ERR_INVALID_ARG, "max_position %d outside [-1, capacity)",
                    max_position);
    int waves, kernel;
    mllm_status st = resolve_opts(opts, &waves, &kernel);
    if (st)
        return st;
    // the slot count covers any wave count up to the option or the maximum
    const int nw = waves > 0 ? waves : MLLM_MAX_WAVES;
    *bytes = mllm::decode_workspace_layout(A, h_q, d.h_kv, d.head_dim, nw).total;
    return ok();
}

}  // extern "C"

namespace {

// Scratch of the allocation-free decode entry point: partial results and the
// plan prefix of a decode call, in place of a caller's workspace.  One copy
// per device, at an address read once per device with hipGetSymbolAddress
// (the array's name in host code is only a stand-in, never a device address);
// every call on a device shares it.
constexpr uint64_t kDecodeScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

// Device address of `scratch` on the current device (which must be `device`).
mllm_status scratch_address(int device, void **ptr)
{
    static std::mutex mu;
    static std::map<int, void *> addr;
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(device);
    if (it == addr.end()) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(decode scratch)");
        if (!p || ((uintptr_t)p) % 256 != 0)
            return fail(MLLM_ERR_DEVICE, "decode scratch has no 256-byte aligned address");
        it = addr.emplace(device, p).first;
    }
    *ptr = it->second;
    return MLLM_OK;
}

// One decode step (mllm_decode_rope_store_attn), its partials in `workspace`
// or, with use_scratch, in this device's `scratch`.
mllm_status decode_impl(mllm_cache *cache, int32_t layer, const mllm_tensor_view *q,
                        const mllm_tensor_view *k_new, const mllm_tensor_view *v_new,
                        const int32_t *positions_dev, const int32_t *cache_rows_dev, int32_t A,
                        const int32_t *host_mirror, const mllm_rope_desc *rope,
                        const mllm_tensor_view *out, void *workspace, uint64_t workspace_bytes,
                        bool use_scratch, int32_t *status_dev, const mllm_decode_opts *opts,
                        void *stream)
{
    if (!cache)
        return fail(MLLM_ERR_INVALID_ARG, "cache is null");
    const mllm_cache_desc &d = cache->desc;
    if (layer < 0 || layer >= d.num_layers)
        return fail(MLLM_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer,
                    d.num_layers);
    if (A < 0)
        return fail(MLLM_ERR_INVALID_ARG, "A must be >= 0 (got %d)", A);
    if (!q)
        return fail(MLLM_ERR_INVALID_ARG, "q view is null");
    if (q->ndim != 3)
        return fail(MLLM_ERR_INVALID_ARG, "q must have 3 dims [A, H_q, D]");
    const int64_t Hq = q->shape[1];
    const int D = d.head_dim;
    if (Hq <= 0 || Hq % d.h_kv != 0)
        return fail(MLLM_ERR_INVALID_ARG, "H_q %lld must be a positive multiple of H_kv %d",
                    (long long)Hq, d.h_kv);
    const int G = (int)(Hq / d.h_kv);
    // the merge and readable launches run one 64-lane wave per (entry, query
    // head), the readable store one 256-lane block per entry
    if (!grid_fits((int64_t)A * Hq, 64) || !grid_fits(A, 256))
        return fail(MLLM_ERR_UNSUPPORTED,
                    "A * H_q = %lld must stay below 2^26 (one 64-lane wave each in a "
                    "one-dimensional grid) and A below 2^24", (long long)A * Hq);
    if (G > 16)
        return fail(MLLM_ERR_UNSUPPORTED, "group size H_q/H_kv = %d exceeds 16", G);
    mllm_status st = check_rope(rope, D);
    if (st)
        return st;
    int waves, kernel;
    st = resolve_opts(opts, &waves, &kernel);
    if (st)
        return st;

    Range rq, rk, rv, ro;
    const int64_t sq[3] = {A, Hq, D}, skv[3] = {A, d.h_kv, D};
    if ((st = check_view(q, "q", 3, sq, d.device, d.dtype, false, &rq)) ||
        (st = check_view(k_new, "k_new", 3, skv, d.device, d.dtype, false, &rk)) ||
        (st = check_view(v_new, "v_new", 3, skv, d.device, d.dtype, false, &rv)) ||
        (st = check_view(out, "out", 3, sq, d.device, d.dtype, true, &ro)))
        return st;
    if (A > 0 && (!positions_dev || !cache_rows_dev))
        return fail(MLLM_ERR_INVALID_ARG, "positions and cache_rows must be non-null");

    if (host_mirror && A > 0) {
        const int32_t *hp = host_mirror, *hr = host_mirror + A;
        std::vector<char> seen(d.slots, 0);
        for (int a = 0; a < A; ++a) {
            if (hp[a] < 0 || hp[a] >= d.capacity)
                return fail(MLLM_ERR_OUT_OF_RANGE, "positions[%d] = %d outside [0, %d)", a,
                            hp[a], d.capacity);
            if (hr[a] < 0 || hr[a] >= d.slots)
                return fail(MLLM_ERR_OUT_OF_RANGE, "cache_rows[%d] = %d outside [0, %d)", a,
                            hr[a], d.slots);
            if (seen[hr[a]])
                return fail(MLLM_ERR_INVALID_ARG, "cache row %d appears twice", hr[a]);
            seen[hr[a]] = 1;
        }
    }
    const int nw_bound = waves > 0 ? waves : MLLM_MAX_WAVES;
    mllm::DecodeWorkspace wl = mllm::decode_workspace_layout(A, Hq, d.h_kv, D, nw_bound);
    if (use_scratch) {
        // the bytes with no partial slot beyond one per (entry, kv head): a
        // lower bound, so a call this rejects needs no device query
        const uint64_t least = mllm::decode_workspace_layout(A, Hq, d.h_kv, D, 0).total;
        if (least > kDecodeScratchBytes)
            return fail(MLLM_ERR_UNSUPPORTED,
                        "A = %d, H_q = %lld needs at least %llu scratch bytes; the "
                        "allocation-free call holds %llu", A, (long long)Hq,
                        (unsigned long long)least, (unsigned long long)kDecodeScratchBytes);
        wl.total = 0;  // library memory: no caller range to check against the others
    } else if (A > 0) {
        if (!workspace)
            return fail(MLLM_ERR_WORKSPACE, "workspace is null");
        if (((uintptr_t)workspace) % 256 != 0)
            return fail(MLLM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (workspace_bytes < wl.total)
            return fail(MLLM_ERR_WORKSPACE, "workspace has %llu bytes, needs %llu",
                        (unsigned long long)workspace_bytes, (unsigned long long)wl.total);
    }
    const uint64_t lb = layer_bytes(d);
    std::vector<Range> ranges = {
        rq, rk, rv, ro,
        Range{"cache K block", (uintptr_t)cache->k[layer], (uintptr_t)cache->k[layer] + lb, true},
        Range{"cache V block", (uintptr_t)cache->v[layer], (uintptr_t)cache->v[layer] + lb, true},
        Range{"workspace", (uintptr_t)workspace, (uintptr_t)workspace + (A ? wl.total : 0), true},
        Range{"positions", (uintptr_t)positions_dev, (uintptr_t)positions_dev + 4u * A, false},
        Range{"cache_rows", (uintptr_t)cache_rows_dev, (uintptr_t)cache_rows_dev + 4u * A, false},
        Range{"status", (uintptr_t)status_dev, (uintptr_t)status_dev + (status_dev ? 4u : 0u),
              true},
    };
    if ((st = check_aliases(ranges)))
        return st;
    if (A == 0)
        return ok();

    // ---- all checks passed: first HIP call from here on
    if ((st = check_device_current(d.device)))
        return st;
    mllm::DecodeParams p;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t *)q->data;
    p.k_new = (const uint16_t *)k_new->data;
    p.v_new = (const uint16_t *)v_new->data;
    p.q_sa = q->stride[0];
    p.q_sh = q->stride[1];
    p.kn_sa = k_new->stride[0];
    p.kn_sh = k_new->stride[1];
    p.vn_sa = v_new->stride[0];
    p.vn_sh = v_new->stride[1];
    p.positions = positions_dev;
    p.rows = cache_rows_dev;
    p.kc = (uint16_t *)cache->k[layer];
    p.vc = (uint16_t *)cache->v[layer];
    p.out = (uint16_t *)out->data;
    p.o_sa = out->stride[0];
    p.o_sh = out->stride[1];
    if (!use_scratch) {
        p.qrot = (float *)((char *)workspace + wl.qrot_off);
        p.part_o = (float *)((char *)workspace + wl.part_o_off);
        p.part_ml = (float *)((char *)workspace + wl.part_ml_off);
        p.plan = (long long *)((char *)workspace + wl.plan_off);
    }
    p.status = status_dev;
    p.A = A;
    p.S = d.slots;
    p.C = d.capacity;
    p.Hq = (int)Hq;
    p.Hkv = d.h_kv;
    p.D = D;
    p.G = G;
    p.HG = mllm::decode_head_group(d.h_kv, G);
    p.NHG = d.h_kv / p.HG;
    p.NS = launch_groups(waves, d.device, D, G, p.HG, d.dtype);
    // the device's resident groups, two per compute unit: the plan gives the
    // first-dispatched half a larger share (see the decode kernel's plan)
    if (use_scratch) {
        // the exact size for the groups this launch runs (NS groups of HG waves)
        wl = mllm::decode_workspace_layout(A, Hq, d.h_kv, D, (int64_t)p.NS * p.HG);
        if (wl.total > kDecodeScratchBytes)
            return fail(MLLM_ERR_UNSUPPORTED,
                        "this decode call needs %llu scratch bytes; the allocation-free call "
                        "holds %llu", (unsigned long long)wl.total,
                        (unsigned long long)kDecodeScratchBytes);
        if ((st = scratch_address(d.device, &workspace)))
            return st;
        p.qrot = (float *)((char *)workspace + wl.qrot_off);
        p.part_o = (float *)((char *)workspace + wl.part_o_off);
        p.part_ml = (float *)((char *)workspace + wl.part_ml_off);
        p.plan = (long long *)((char *)workspace + wl.plan_off);
    }
    p.plan_weighted = waves == 0 && p.NS == 2 * device_cus(d.device) ? 1 : 0;
    // more query heads per kv head, more work per tile: a different lead of the
    // first-dispatched groups (ratios measured on MI355X)
    p.plan_wa = G <= 4 ? 46 : 45;
    p.plan_wb = G <= 4 ? 30 : 28;
    p.dtype = d.dtype;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    fill_inv_freq(p.inv_freq, rope->base, D);

    hipStream_t s = (hipStream_t)stream;
    hipEvent_t *ev = opts ? (hipEvent_t *)opts->attn_events : nullptr;
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    hipError_t e;
    if (kernel == 1) {  // readable path: a store kernel, then one wave per query head
        e = mllm::launch_rope_store(p, s);
        if (e != hipSuccess)
            return hip_fail(e, "rope/store launch");
        e = mllm::launch_decode_readable(p, s, e0, e1);
    } else {
        e = mllm::launch_decode_fused(p, s, e0, e1);
        if (e == hipSuccess)
            e = mllm::launch_decode_merge(p, s);
    }
    if (e != hipSuccess)
        return hip_fail(e, "attention launch");
    if (host_mirror) {
        for (int a = 0; a < A; ++a) {
            const int32_t r = host_mirror[A + a], pos = host_mirror[a];
            if (cache->length[r] < pos + 1)
                cache->length[r] = pos + 1;
        }
    }
    return ok();
}

}  // namespace

extern "C" {

mllm_status mllm_decode_rope_store_attn(mllm_cache *cache, int32_t layer,
                                        const mllm_tensor_view *q,
                                        const mllm_tensor_view *k_new,
                                        const mllm_tensor_view *v_new,
                                        const int32_t *positions_dev,
                                        const int32_t *cache_rows_dev, int32_t A,
                                        const int32_t *host_mirror,
                                        const mllm_rope_desc *rope,
                                        const mllm_tensor_view *out, void *workspace,
                                        uint64_t workspace_bytes, int32_t *status_dev,
                                        const mllm_decode_opts *opts, void *stream)
{
    return decode_impl(cache, layer, q, k_new, v_new, positions_dev, cache_rows_dev, A,
                       host_mirror, rope, out, workspace, workspace_bytes, false, status_dev,
                       opts, stream);
}

mllm_status mllm_decode_rope_store_attn_noalloc(mllm_cache *cache, int32_t layer,
                                                const mllm_tensor_view *q,
                                                const mllm_tensor_view *k_new,
                                                const mllm_tensor_view *v_new,
                                                const int32_t *positions_dev,
                                                const int32_t *cache_rows_dev, int32_t A,
                                                const int32_t *host_mirror,
                                                const mllm_rope_desc *rope,
                                                const mllm_tensor_view *out,
                                                int32_t *status_dev,
                                                const mllm_decode_opts *opts, void *stream)
{
    return decode_impl(cache, layer, q, k_new, v_new, positions_dev, cache_rows_dev, A,
                       host_mirror, rope, out, nullptr, 0, true, status_dev, opts, stream);
}

mllm_status mllm_prefill_workspace_size(const mllm_cache *cache, int32_t A, int32_t T,
                                        int32_t h_q, uint64_t *bytes)
{
    if (!cache || !bytes)
        return fail(MLLM_ERR_INVALID_ARG, "cache and bytes must be non-null");
    const mllm_cache_desc &d = cache->desc;
    if (A < 0 || T < 1 || T > d.capacity)
        return fail(MLLM_ERR_INVALID_ARG, "need A >= 0 and 1 <= T <= capacity");
    if (h_q <= 0 || h_q % d.h_kv != 0)
        return fail(MLLM_ERR_INVALID_ARG, "h_q %d must be a positive multiple of h_kv %d", h_q,
                    d.h_kv);
    *bytes = mllm::prefill_workspace_bytes(A, T, h_q, d.head_dim);
    return ok();
}

}  // extern "C"

namespace {

// Both prefill calls: chunk_host == NULL is the equal-length prefill into
// empty rows (rows_host, starts 0, lengths T); otherwise chunk_host holds
// {starts, lengths, rows} of A entries and chunk_dev the same on the device.
mllm_status prefill_call(mllm_cache *cache, int32_t layer, const mllm_tensor_view *q,
                         const mllm_tensor_view *k_new, const mllm_tensor_view *v_new,
                         const int32_t *rows_dev, const int32_t *rows_host,
                         const int32_t *chunk_dev, const int32_t *chunk_host, int32_t A,
                         int32_t T, const mllm_rope_desc *rope, const mllm_tensor_view *out,
                         void *workspace, uint64_t workspace_bytes, const mllm_decode_opts *opts,
                         void *stream)
{
    if (!cache)
        return fail(MLLM_ERR_INVALID_ARG, "cache is null");
    const mllm_cache_desc &d = cache->desc;
    const bool chunk = chunk_host != nullptr || chunk_dev != nullptr;
    if (layer < 0 || layer >= d.num_layers)
        return fail(MLLM_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer,
                    d.num_layers);
    if (A < 0)
        return fail(MLLM_ERR_INVALID_ARG, "A must be >= 0 (got %d)", A);
    if (T < 1 || T > d.capacity)
        return fail(MLLM_ERR_INVALID_ARG, "T = %d outside [1, capacity = %d]", T, d.capacity);
    if (!q)
        return fail(MLLM_ERR_INVALID_ARG, "q view is null");
    if (q->ndim != 4)
        return fail(MLLM_ERR_INVALID_ARG, "q must have 4 dims [A, T, H_q, D]");
    const int64_t Hq = q->shape[2];
    const int D = d.head_dim;
    if (Hq <= 0 || Hq % d.h_kv != 0)
        return fail(MLLM_ERR_INVALID_ARG, "H_q %lld must be a positive multiple of H_kv %d",
                    (long long)Hq, d.h_kv);
    const int G = (int)(Hq / d.h_kv);
    mllm_status st = check_rope(rope, D);
    if (st)
        return st;
    int waves_unused, kernel;
    if ((st = resolve_opts(opts, &waves_unused, &kernel)))
        return st;
    // one-dimensional grids: the store kernel one 64-lane wave per (entry,
    // token), the matrix-core kernel one 256-lane block per (entry, group of
    // HB query heads, 128 / HB queries) -- at most one per (entry, query head,
    // 128 queries), the bound checked here --, the readable kernel one 64-lane
    // wave per (entry, token, query head)
    if (!grid_fits((int64_t)A * T, 64) ||
        (kernel == 1 ? !grid_fits((int64_t)A * T * Hq, 64)
                     : !grid_fits((int64_t)A * Hq * ((T + 127) / 128), 256)))
        return fail(MLLM_ERR_UNSUPPORTED,
                    "A = %d, T = %d, H_q = %lld exceed a one-dimensional launch grid "
                    "(2^32 work-items)", A, T, (long long)Hq);
    Range rq, rk, rv, ro;
    const int64_t sq[4] = {A, T, Hq, D}, skv[4] = {A, T, d.h_kv, D};
    if ((st = check_view(q, "q", 4, sq, d.device, d.dtype, false, &rq)) ||
        (st = check_view(k_new, "k_new", 4, skv, d.device, d.dtype, false, &rk)) ||
        (st = check_view(v_new, "v_new", 4, skv, d.device, d.dtype, false, &rv)) ||
        (st = check_view(out, "out", 4, sq, d.device, d.dtype, true, &ro)))
        return st;
    if (chunk) {
        if (A > 0 && (!chunk_dev || !chunk_host))
            return fail(MLLM_ERR_INVALID_ARG, "chunk metadata (device and host) must be non-null");
        rows_dev = chunk_dev ? chunk_dev + 2 * A : nullptr;
        rows_host = chunk_host ? chunk_host + 2 * A : nullptr;
    } else if (A > 0 && (!rows_dev || !rows_host)) {
        return fail(MLLM_ERR_INVALID_ARG, "cache_rows (device and host) must be non-null");
    }
    std::vector<char> seen(d.slots, 0);
    for (int a = 0; a < A; ++a) {
        const int r = rows_host[a];
        if (r < 0 || r >= d.slots)
            return fail(MLLM_ERR_OUT_OF_RANGE, "cache_rows[%d] = %d outside [0, %d)", a, r,
                        d.slots);
        if (seen[r])
            return fail(MLLM_ERR_INVALID_ARG, "cache row %d appears twice", r);
        seen[r] = 1;
        if (!chunk) {
            if (cache->length[r] != 0)
                return fail(MLLM_ERR_ROW_BUSY, "cache row %d is not empty (length %d); reset "
                            "it first", r, cache->length[r]);
            continue;
        }
        const int s0 = chunk_host[a], n = chunk_host[A + a];
        if (n < 1 || n > T)
            return fail(MLLM_ERR_INVALID_ARG, "lengths[%d] = %d outside [1, T = %d]", a, n, T);
        if (s0 < 0)
            return fail(MLLM_ERR_OUT_OF_RANGE, "starts[%d] = %d is negative", a, s0);
        if (s0 > d.capacity - n)
            return fail(MLLM_ERR_OUT_OF_RANGE, "starts[%d] + lengths[%d] = %d exceeds capacity %d",
                        a, a, s0 + n, d.capacity);
    }
    const uint64_t need = mllm::prefill_workspace_bytes(A, T, Hq, D);
    if (A > 0 && need > 0) {
        if (!workspace)
            return fail(MLLM_ERR_WORKSPACE, "workspace is null");
        if (((uintptr_t)workspace) % 256 != 0)
            return fail(MLLM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (workspace_bytes < need)
            return fail(MLLM_ERR_WORKSPACE, "workspace has %llu bytes, needs %llu",
                        (unsigned long long)workspace_bytes, (unsigned long long)need);
    }
    const uint64_t lb = layer_bytes(d);
    const uintptr_t meta = chunk ? (uintptr_t)chunk_dev : (uintptr_t)rows_dev;
    std::vector<Range> ranges = {
        rq, rk, rv, ro,
        Range{"cache K block", (uintptr_t)cache->k[layer], (uintptr_t)cache->k[layer] + lb, true},
        Range{"cache V block", (uintptr_t)cache->v[layer], (uintptr_t)cache->v[layer] + lb, true},
        Range{"workspace", (uintptr_t)workspace, (uintptr_t)workspace + (A ? need : 0), true},
        Range{chunk ? "chunk metadata" : "cache_rows", meta,
              meta + (chunk ? 12u : 4u) * (uintptr_t)A, false},
    };
    if ((st = check_aliases(ranges)))
        return st;
    if (A == 0)
        return ok();

    if ((st = check_device_current(d.device)))
        return st;
    mllm::PrefillParams p;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t *)q->data;
    p.k_new = (const uint16_t *)k_new->data;
    p.v_new = (const uint16_t *)v_new->data;
    p.q_sa = q->stride[0];
    p.q_st = q->stride[1];
    p.q_sh = q->stride[2];
    p.kn_sa = k_new->stride[0];
    p.kn_st = k_new->stride[1];
    p.kn_sh = k_new->stride[2];
    p.vn_sa = v_new->stride[0];
    p.vn_st = v_new->stride[1];
    p.vn_sh = v_new->stride[2];
    p.rows = rows_dev;
    p.starts = chunk ? chunk_dev : nullptr;
    p.lens = chunk ? chunk_dev + A : nullptr;
    p.kc = (uint16_t *)cache->k[layer];
    p.vc = (uint16_t *)cache->v[layer];
    p.out = (uint16_t *)out->data;
    p.o_sa = out->stride[0];
    p.o_st = out->stride[1];
    p.o_sh = out->stride[2];
    p.table = (float2 *)workspace;
    p.A = A;
    p.T = T;
    p.S = d.slots;
    p.C = d.capacity;
    p.Hq = (int)Hq;
    p.Hkv = d.h_kv;
    p.D = D;
    p.G = G;
    p.dtype = d.dtype;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    fill_inv_freq(p.inv_freq, rope->base, D);
    mllm::prefill_order(p, chunk ? chunk_host : nullptr, chunk ? chunk_host + A : nullptr);
    hipEvent_t *ev = opts ? (hipEvent_t *)opts->attn_events : nullptr;
    hipError_t e = mllm::launch_prefill(p, (hipStream_t)stream, kernel, ev ? ev[0] : nullptr,
                                        ev ? ev[1] : nullptr);
    if (e != hipSuccess)
        return hip_fail(e, "prefill launch");
    for (int a = 0; a < A; ++a) {
        const int r = rows_host[a];
        const int end = chunk ? chunk_host[a] + chunk_host[A + a] : T;
        if (cache->length[r] < end)
            cache->length[r] = end;
    }
    return ok();
}

}  // namespace

extern "C" {

mllm_status mllm_prefill_rope_store_attn(mllm_cache *cache, int32_t layer,
                                         const mllm_tensor_view *q,
                                         const mllm_tensor_view *k_new,
                                         const mllm_tensor_view *v_new,
                                         const int32_t *cache_rows_dev,
                                         const int32_t *cache_rows_host, int32_t A, int32_t T,
                                         const mllm_rope_desc *rope,
                                         const mllm_tensor_view *out, void *workspace,
                                         uint64_t workspace_bytes, const mllm_decode_opts *opts,
                                         void *stream)
{
    return prefill_call(cache, layer, q, k_new, v_new, cache_rows_dev, cache_rows_host, nullptr,
                        nullptr, A, T, rope, out, workspace, workspace_bytes, opts, stream);
}

mllm_status mllm_prefill_chunk_rope_store_attn(mllm_cache *cache, int32_t layer,
                                               const mllm_tensor_view *q,
                                               const mllm_tensor_view *k_new,
                                               const mllm_tensor_view *v_new,
                                               const int32_t *chunk_dev,
                                               const int32_t *chunk_host, int32_t A, int32_t T,
                                               const mllm_rope_desc *rope,
                                               const mllm_tensor_view *out, void *workspace,
                                               uint64_t workspace_bytes,
                                               const mllm_decode_opts *opts, void *stream)
{
    if (A > 0 && (!chunk_dev || !chunk_host))
        return fail(MLLM_ERR_INVALID_ARG, "chunk metadata (device and host) must be non-null");
    return prefill_call(cache, layer, q, k_new, v_new, nullptr, nullptr, chunk_dev, chunk_host,
                        A, T, rope, out, workspace, workspace_bytes, opts, stream);
}

}  // extern "C"
