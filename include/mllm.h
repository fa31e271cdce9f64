/*
 * mllm.h -- C ABI of the positions-aware cached decode library for MI355X
 * (gfx950).  ABI version 1.
 *
 * The operation (microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary"):
 * survivor tokens keep fixed cache-row IDs; device tensors positions[A] and
 * cache_rows[A] parameterize decode-only RoPE, the K/V store and cached
 * attention, and inactive full-capacity rows stay untouched.  Equal-length
 * pending prompts are prefilled as one batch whose prefixes land in empty
 * shared rows.
 *
 * Boundary conventions (ARCHITECTURE.md, "Tensor ownership boundary" and
 * "Stable integration boundary"):
 *  - tensors cross as non-owning views: pointer, accessible bytes, shape,
 *    element strides, dtype and device; the caller keeps ownership;
 *  - output, workspace, device and stream are explicit; nothing is inferred
 *    from a pointer; unsupported layouts are rejected, never copied behind the
 *    caller's back;
 *  - no entry point throws; each returns an mllm_status and records a
 *    thread-local message readable through mllm_last_error();
 *  - every argument check runs before the first HIP call, and a call that
 *    fails a check has no side effect;
 *  - the compute calls never allocate, never synchronize and run only on the
 *    given stream.
 *
 * Layouts (all in the cache's storage type, BF16 or FP16; element strides,
 * innermost dimension contiguous).  rnd(x) below is x rounded to that type
 * (nearest, ties to even):
 *  cache K, V : [slots, capacity, H_kv, D] per layer, dense
 *  decode  q  : [A, H_q, D]      k_new, v_new : [A, H_kv, D]    out : [A, H_q, D]
 *  prefill q  : [A, T, H_q, D]   k_new, v_new : [A, T, H_kv, D] out : [A, T, H_q, D]
 * Query head hq reads kv head hq / (H_q / H_kv).
 */
#ifndef MLLM_H
#define MLLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLLM_ABI_VERSION 1

typedef enum {
    MLLM_OK = 0,
    MLLM_ERR_INVALID_ARG = 1,  /* null pointer, bad shape/stride/size, out-of-range index */
    MLLM_ERR_UNSUPPORTED = 2,  /* dtype, head size or layout the library does not handle */
    MLLM_ERR_ALIAS = 3,        /* a writable buffer overlaps another argument */
    MLLM_ERR_OUT_OF_RANGE = 4, /* position or row outside the cache (host mirror check) */
    MLLM_ERR_ROW_BUSY = 5,     /* prefill target row is not logically empty */
    MLLM_ERR_WORKSPACE = 6,    /* workspace null or smaller than the *_workspace_size value */
    MLLM_ERR_OUT_OF_MEMORY = 7,
    MLLM_ERR_DEVICE = 8        /* a HIP runtime call failed; see mllm_last_error() */
} mllm_status;

/* Storage type of the cache and of every 16-bit tensor of a call (the typed
 * FP16/BF16 softmax of operator-development.md, "Public interfaces"): one
 * type per cache, and each view of a call must carry the cache's type. */
typedef enum { MLLM_BF16 = 1, MLLM_F16 = 2 } mllm_dtype;

/*
 * Non-owning tensor view ("Tensor ownership boundary": the C ABI builds a
 * non-owning view from pointer, accessible bytes, shape, element strides,
 * dtype and device).  Elements [i0..] live at data + sum(i_k * stride[k]) *
 * element size; every such address must fall inside [data, data + bytes).
 * Negative dims or strides are rejected.  Zero-size dims are legal.
 */
typedef struct {
    void *data;
    uint64_t bytes;
    int32_t ndim;
    int32_t dtype;     /* mllm_dtype */
    int32_t device;    /* HIP device ordinal */
    int32_t reserved;
    int64_t shape[4];
    int64_t stride[4]; /* in elements */
} mllm_tensor_view;

/* Shared slot cache: num_layers x {K, V} x [slots, capacity, h_kv, head_dim]. */
typedef struct {
    int32_t num_layers;
    int32_t slots;
    int32_t capacity;  /* positions per row: the persistent bound on sequence length */
    int32_t h_kv;
    int32_t head_dim;  /* 64 or 128 */
    int32_t dtype;     /* MLLM_BF16 or MLLM_F16 */
    int32_t device;
} mllm_cache_desc;

/* Split-half RoPE over the whole head ("Attention layout boundary"): pairs
 * (i, i + D/2), angle pos * base^(-2i/D); base must be finite and > 0. */
typedef struct {
    double base;
    int32_t rotary_dim; /* must equal head_dim */
    int32_t reserved;
} mllm_rope_desc;

/* Optional knobs of the decode and prefill calls (NULL = defaults). */
typedef struct {
    /* Decode: waves that share the 32-key tiles of all (entry, kv head)
     * segments.  Waves run in groups of up to 8, one per kv head of a head
     * group, and each group takes an equal share of the (entry, key tile)
     * columns.  0 = the device's resident groups; else 1 .. MLLM_MAX_WAVES,
     * rounded down to whole groups (at least one).  The output bits depend on
     * this count.  Ignored by prefill. */
    int32_t waves;
    int32_t kernel;         /* 0 = tuned kernels, 1 = readable one-wave-per-head kernel */
    /* NULL, or a hipEvent_t[2] that the call stamps at the start and the end
     * of the attention kernel (the tuned kernel, or the readable
     * kernel), for per-kernel timing attribution (operator-development.md,
     * "Public interfaces": Event timing attributed per layer). */
    void *attn_events;
    int32_t reserved[4];
} mllm_decode_opts;

#define MLLM_MAX_WAVES 4096

typedef struct mllm_cache mllm_cache; /* opaque */

/* ABI version of the loaded library (MLLM_ABI_VERSION): the C ABI is versioned
 * ("Stable integration boundary": the seam is a C-compatible descriptor with
 * explicit stream and workspace, and the C ABI carries a version). */
int mllm_abi_version(void);

/* Thread-local text of the last failure on this thread ("" after success):
 * every rejected call fails explicitly with a status and this message ("Tensor
 * N0 invariants": unsupported operations fail explicitly). */
const char *mllm_last_error(void);

/* Exact device bytes of a cache: num_layers * 2 * slots * capacity * h_kv *
 * head_dim * 2 ("Tensor ownership boundary": serving runners verify the exact
 * layer/head/element-size allocation formula). */
mllm_status mllm_cache_bytes(const mllm_cache_desc *desc, uint64_t *bytes);

/* Allocate an engine-owned cache with hipMalloc on desc->device ("Tensor
 * ownership boundary": a shared cache allocation that persists while rows come
 * and go; the same kernels consume engine-owned or caller-owned memory).
 * Contents are not initialized; every row starts logically empty (length 0). */
mllm_status mllm_cache_alloc(const mllm_cache_desc *desc, mllm_cache **out);

/* Wrap caller-owned device memory (e.g. torch tensors) as a cache ("Tensor
 * ownership boundary": ownership is never inferred from a pointer, so the same
 * kernels run on engine-owned or PyTorch-owned allocations).  k_layers
 * and v_layers hold num_layers pointers, each to a dense [slots, capacity,
 * h_kv, head_dim] block of desc->dtype, 16-byte aligned.  The caller keeps ownership and
 * must keep the memory alive until mllm_cache_free. */
mllm_status mllm_cache_wrap(const mllm_cache_desc *desc, void *const *k_layers,
                            void *const *v_layers, mllm_cache **out);

/* Release the cache object, and its memory if engine-owned ("Tensor ownership
 * boundary": storage owns an allocation, views do not).  NULL is a no-op. */
mllm_status mllm_cache_free(mllm_cache *cache);

/* Device pointers of one layer's K and V blocks: non-owning, valid while the
 * cache lives ("Tensor ownership boundary": views are non-owning). */
mllm_status mllm_cache_layer(const mllm_cache *cache, int32_t layer, void **k, void **v);

/* Copy of the descriptor the cache was created with ("Stable integration
 * boundary": the cache crosses the ABI as a C descriptor). */
mllm_status mllm_cache_get_desc(const mllm_cache *cache, mllm_cache_desc *desc);

/* Logical reset of one row ("Tensor ownership boundary": the shared allocation
 * persists while a finished row's active prefix falls to zero; a reset row is
 * reused from position zero).  Sets the row length to 0; touches no device
 * memory. */
mllm_status mllm_cache_reset_row(mllm_cache *cache, int32_t row);

/* Host-side logical length of one row ("Tensor ownership boundary": a row's
 * active prefix grows with its decode steps and falls to zero on reset): T after
 * a prefill, max(len, pos + 1) after a decode made with a host mirror, 0 after a
 * reset. */
mllm_status mllm_cache_row_length(const mllm_cache *cache, int32_t row, int32_t *len);

/* Declare a row's logical length, 0 <= len <= capacity (MLLM_ERR_OUT_OF_RANGE
 * otherwise): for a caller that filled or restored the row by other means, or
 * decoded without a host mirror ("Tensor ownership boundary": the scheduler
 * above the model primitives owns each row's state).  Touches no device
 * memory. */
mllm_status mllm_cache_set_row_length(mllm_cache *cache, int32_t row, int32_t len);

/* Workspace bytes needed by mllm_decode_rope_store_attn for A entries and h_q
 * query heads with the given opts (may be NULL) ("Stable integration
 * boundary": the workspace is explicit and caller-owned).  max_position bounds every
 * position of the call (-1 = capacity - 1); the current layout's size does not
 * depend on it.  The size is the same for every position, so one workspace serves
 * every step of a decode loop. */
mllm_status mllm_decode_workspace_size(const mllm_cache *cache, int32_t A, int32_t h_q,
                                       int32_t max_position, const mllm_decode_opts *opts,
                                       uint64_t *bytes);

/*
 * One decode step of one layer ("Tensor ownership boundary": device
 * positions[A] and cache_rows[A] parameterize decode RoPE, the K/V store and
 * cached attention; inactive rows untouched).  For every a < A, with
 * p = positions[a], r = cache_rows[a], on `stream`:
 *   1. K[r, p, h, :] = rnd(RoPE(k_new[a, h, :], p)) and V[r, p, h, :] =
 *      v_new[a, h, :] (bit copy) for every kv head h; no other cache byte is
 *      written;
 *   2. out[a, hq, :] = rnd( softmax_j( RoPE(q[a, hq], p) . K[r, j, hq/G] /
 *      sqrt(D) ) . V[r, j, hq/G] ) over j = 0..p, the softmax reduced in FP32
 *      and only the output rounded (operator-development.md, "Public
 *      interfaces": typed softmax reduces in FP32 registers).
 *
 *  q, k_new, v_new : device views, layouts above; D contiguous, 16-byte aligned
 *                    rows; any non-negative outer strides.
 *  positions_dev, cache_rows_dev : device int32[A].
 *  host_mirror     : NULL, or host int32[2*A] = {positions[0..A), rows[0..A)},
 *                    the same values as the device arrays.  With it the call
 *                    also rejects out-of-range positions/rows and duplicate
 *                    rows (MLLM_ERR_OUT_OF_RANGE / MLLM_ERR_INVALID_ARG) and
 *                    updates the row lengths.  Without it the kernels skip the
 *                    store for an out-of-range entry, write NaN to its output
 *                    and set *status_dev to 1; duplicate rows are then the
 *                    caller's error (two stores race).
 *  out             : device view [A, H_q, D]; must not overlap any input,
 *                    the cache or the workspace (MLLM_ERR_ALIAS).
 *  workspace       : device buffer of at least mllm_decode_workspace_size()
 *                    bytes (same A, h_q and opts), 256-byte aligned,
 *                    caller-owned, contents ignored on entry (the call writes
 *                    partial results there).  One workspace serves one call
 *                    at a time: calls that overlap in time need distinct
 *                    workspaces.
 *  status_dev      : NULL or device int32, set to 1 on a device-side index
 *                    error, never cleared by the library.
 *  stream          : hipStream_t (NULL = the null stream).
 *  A = 0 is a successful no-op; A * h_q must stay below 2^31
 *  (MLLM_ERR_UNSUPPORTED).  The call is idempotent (same inputs give the same
 *  cache bytes and output bits).
 */
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
                                        const mllm_decode_opts *opts, void *stream);

/*
 * The decode step of mllm_decode_rope_store_attn without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * partial results and the plan live in a scratch array of the library
 * (64 MiB per device, held from the first call on a device until the process
 * ends); the call allocates nothing.  Arguments, results, checks and errors are
 * those of mllm_decode_rope_store_attn, with the same output bits for the same
 * inputs and options.  A call that needs more scratch than 64 MiB (about
 * A * H_q * D * 4 + (A * H_kv + waves of the launch) * G * (D + 2) * 4 bytes)
 * returns MLLM_ERR_UNSUPPORTED before any launch.  Every call on one device
 * shares that device's scratch: calls that overlap in time on one device race
 * (run them on one stream, or one at a time).
 */
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
                                                const mllm_decode_opts *opts, void *stream);

/* Workspace bytes needed by mllm_prefill_rope_store_attn and
 * mllm_prefill_chunk_rope_store_attn for A entries of (up to) T tokens and
 * h_q query heads: a cos/sin table of A * T * head_dim / 2 float pairs
 * ("Stable integration boundary": the workspace is explicit and caller-owned). */
mllm_status mllm_prefill_workspace_size(const mllm_cache *cache, int32_t A, int32_t T,
                                        int32_t h_q, uint64_t *bytes);

/*
 * Equal-length batched prefill of one layer ("Tensor ownership boundary":
 * equal-length pending prompts run as one batch and each prefix is mapped
 * into its target empty shared-cache row; different lengths are separate
 * calls).  For every a < A and t < T, with r = cache_rows[a]:
 *   K[r, t, h, :] = rnd(RoPE(k_new[a, t, h, :], t)), V[r, t, h, :] = v_new[a, t, h, :];
 *   out[a, t, hq, :] = causal GQA attention of RoPE(q[a, t, hq], t) over keys
 *   0..t of row r, FP32 softmax, output rounded to the storage type.  The
 *   attention products run on the matrix cores in the storage type: the FP32
 *   rotated query enters as two parts (high part and rounded remainder:
 *   2^-16 relative for BF16, 2^-22 for FP16), the softmax weights (in [0, 1])
 *   are rounded to the storage type once, accumulation is FP32.
 * Positions >= T of row r and every other row stay untouched.
 *
 *  cache_rows_dev  : device int32[A]; cache_rows_host: host int32[A], the
 *                    same values (required: rows are checked in range,
 *                    distinct and logically empty, else MLLM_ERR_ROW_BUSY).
 *  1 <= T <= capacity; A * T * H_q must stay below 2^31 (MLLM_ERR_UNSUPPORTED).
 *  On success every target row's length becomes T.
 *  opts (may be NULL): kernel 0 = matrix-core kernel, 1 = readable kernel;
 *  attn_events timestamps the attention kernel; waves is ignored.
 *  Other arguments as for the decode call.
 */
mllm_status mllm_prefill_rope_store_attn(mllm_cache *cache, int32_t layer,
                                         const mllm_tensor_view *q,
                                         const mllm_tensor_view *k_new,
                                         const mllm_tensor_view *v_new,
                                         const int32_t *cache_rows_dev,
                                         const int32_t *cache_rows_host, int32_t A, int32_t T,
                                         const mllm_rope_desc *rope,
                                         const mllm_tensor_view *out, void *workspace,
                                         uint64_t workspace_bytes, const mllm_decode_opts *opts,
                                         void *stream);

/*
 * Prefill chunk of one layer appended at per-entry start positions, with
 * per-entry lengths.  The pages define the equal-length prefill into empty
 * rows and the one-token cached decode step, and keep prompts of different
 * lengths as separate groups ("Tensor ownership boundary"); this call reads a
 * chunk of n tokens at start s as n decode steps at positions s .. s+n-1
 * taken together, and a batch of several lengths as those equal-length groups
 * run one after another.  For every a < A, with s = starts[a],
 * n = lengths[a], r = rows[a], and every t < n:
 *   K[r, s+t, h, :] = rnd(RoPE(k_new[a, t, h, :], s+t)),
 *   V[r, s+t, h, :] = v_new[a, t, h, :];
 *   out[a, t, hq, :] = causal GQA attention of RoPE(q[a, t, hq], s+t) over
 *   keys 0..s+t of row r (the cached prefix and the chunk up to t), FP32
 *   softmax, rounded output; the products run on the matrix cores as in
 *   mllm_prefill_rope_store_attn.
 * Tokens t >= n of an entry are ignored and out[a, t] is not written; no
 * other cache byte is written.  starts 0 and lengths T on empty rows give
 * exactly mllm_prefill_rope_store_attn.
 *
 *  chunk_dev   : device int32[3*A] = {starts[0..A), lengths[0..A),
 *                rows[0..A)}: one array, as the page moves token, position
 *                and row metadata in one [3, A] transfer.
 *  chunk_host  : host int32[3*A], the same values (required).  Rows must be
 *                in range (MLLM_ERR_OUT_OF_RANGE) and distinct
 *                (MLLM_ERR_INVALID_ARG); 1 <= lengths[a] <= T
 *                (MLLM_ERR_INVALID_ARG); 0 <= starts[a] and starts[a] +
 *                lengths[a] <= capacity (MLLM_ERR_OUT_OF_RANGE).  Slots
 *                0 .. starts[a]-1 of the row are read as the cached prefix
 *                whatever the row's recorded length (as the decode call reads
 *                0 .. position).  Nothing is launched when a check fails.
 *                Device values that
 *                disagree with the host copy make the kernels skip that
 *                entry's stores and write NaN to its T output rows.
 *  q [A, T, H_q, D], k_new / v_new [A, T, H_kv, D], out [A, T, H_q, D]:
 *                T is the longest length of the batch, 1 <= T <= capacity.
 *  workspace   : at least mllm_prefill_workspace_size(A, T, h_q) bytes.
 *  On success each row's length becomes max(length, starts[a] + lengths[a]).
 *  opts and the other arguments as for mllm_prefill_rope_store_attn.
 */
mllm_status mllm_prefill_chunk_rope_store_attn(mllm_cache *cache, int32_t layer,
                                               const mllm_tensor_view *q,
                                               const mllm_tensor_view *k_new,
                                               const mllm_tensor_view *v_new,
                                               const int32_t *chunk_dev,
                                               const int32_t *chunk_host, int32_t A, int32_t T,
                                               const mllm_rope_desc *rope,
                                               const mllm_tensor_view *out, void *workspace,
                                               uint64_t workspace_bytes,
                                               const mllm_decode_opts *opts, void *stream);

/* ---------------------------------------------------------------------------
 * Slot manager ("Tensor ownership boundary": a scheduler above the model
 * primitives owns the request-to-row map, admits only at step boundaries,
 * resets a row on length, stop or cancel and reuses the lowest free slot; the
 * shared cache allocation persists while the rows' active prefixes fall back
 * to zero; max_sequence_length bounds the persistent cache, zero keeping the
 * model maximum).  Host logic over the calls above: it reads the rows'
 * logical lengths, which the prefill and decode calls advance (the decode call
 * with a host mirror), resets rows logically, and makes no device call.  One
 * thread at a time per scheduler; the scheduler owns every row of its cache.
 */
typedef struct mllm_sched mllm_sched;

/* Why a request left its row. */
typedef enum { MLLM_END_LENGTH = 1, MLLM_END_STOP = 2, MLLM_END_CANCEL = 3 } mllm_end;

/* One line of a step plan. */
typedef struct {
    int64_t request_id;
    int32_t row;
    int32_t value; /* admitted: prompt length; decode: the position the request's
                      next token is stored at (the row's length); retired: mllm_end */
} mllm_sched_entry;

/* A scheduler over every row of `cache` ("Tensor ownership boundary": the
 * scheduler owns the request-to-row map); each row must be empty (length 0,
 * else MLLM_ERR_ROW_BUSY).  max_sequence_length: 0 = the cache capacity,
 * else 1..capacity (MLLM_ERR_OUT_OF_RANGE; the same section bounds the
 * persistent cache by it, zero keeping the model maximum). */
mllm_status mllm_sched_create(mllm_cache *cache, int32_t max_sequence_length, mllm_sched **out);
/* Release the scheduler (not the cache: "Tensor ownership boundary", the shared
 * cache allocation persists). */
mllm_status mllm_sched_free(mllm_sched *sched);
/* The bound in force, the cache capacity when created with 0 ("Tensor ownership
 * boundary": max_sequence_length bounds the persistent cache). */
mllm_status mllm_sched_max_sequence_length(const mllm_sched *sched, int32_t *len);

/* Queue a request, first in first out; it is admitted at a later step boundary
 * ("Tensor ownership boundary": admission only at scheduler-step boundaries).
 * prompt_len >= 1, max_new_tokens >= 0
 * (MLLM_ERR_INVALID_ARG); prompt_len + max_new_tokens <= max_sequence_length
 * (MLLM_ERR_OUT_OF_RANGE); ids unique among queued and active requests
 * (MLLM_ERR_INVALID_ARG). */
mllm_status mllm_sched_submit(mllm_sched *sched, int64_t request_id, int32_t prompt_len,
                              int32_t max_new_tokens);
/* End a request ("Tensor ownership boundary": a row is reset on length, stop or
 * cancel): stop (the caller saw its stop token) takes effect at the next
 * boundary; cancel removes a queued request at once and ends an active one at
 * the next boundary.  Unknown id: MLLM_ERR_INVALID_ARG. */
mllm_status mllm_sched_stop(mllm_sched *sched, int64_t request_id);
mllm_status mllm_sched_cancel(mllm_sched *sched, int64_t request_id);

/*
 * Step boundary ("Tensor ownership boundary": admission only at step
 * boundaries, reset on length/stop/cancel, the lowest free slot reused).  In
 * order:
 *  1. retire: each active request that was cancelled (MLLM_END_CANCEL) or
 *     stopped (MLLM_END_STOP), or whose row holds prompt_len + max_new_tokens
 *     positions (MLLM_END_LENGTH; each decode step stores one token), leaves
 *     its row; the row is reset to length 0 and freed;
 *  2. decode: every request admitted at an earlier boundary that remains, by
 *     row, with the position its next token is stored at (the row's length);
 *  3. admit: queued requests, first in first out, take the lowest free rows
 *     while any is free; listed by prompt length, then row, so equal prompt
 *     lengths are contiguous (one equal-length prefill group each, or one
 *     prefill chunk call for all).  They decode from the next boundary on.
 * The caller then runs this step: the prefill of the admitted rows and the
 * decode of the decode list (with a host mirror, so the row lengths advance).
 * Each array is caller-owned with room for at least `slots` entries
 * (MLLM_ERR_INVALID_ARG otherwise, nothing changed).
 */
mllm_status mllm_sched_boundary(mllm_sched *sched, mllm_sched_entry *admitted,
                                int32_t admitted_cap, int32_t *n_admitted,
                                mllm_sched_entry *decode, int32_t decode_cap, int32_t *n_decode,
                                mllm_sched_entry *retired, int32_t retired_cap,
                                int32_t *n_retired);
/* Requests waiting in the queue and requests holding a row ("Tensor ownership
 * boundary": the scheduler exposes snapshots of its state). */
mllm_status mllm_sched_counts(const mllm_sched *sched, int32_t *queued, int32_t *active);

#ifdef __cplusplus
}
#endif

#endif /* MLLM_H */
