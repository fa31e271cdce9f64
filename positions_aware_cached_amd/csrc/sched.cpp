// sched.cpp -- the slot manager of the C ABI (mllm_sched_*).
//
// microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary": a scheduler
// above the model primitives owns the request-to-row map; it admits only at
// step boundaries, resets a row on length / stop / cancel and reuses the
// lowest free slot, and the shared cache allocation persists while the rows'
// active prefixes fall back to zero.  The same page bounds the persistent cache
// by max_sequence_length (zero keeps the model maximum, a positive value must
// fit the model and every submitted request).
//
// Host logic only, written over the public cache calls: it reads the rows'
// logical lengths (which the prefill and decode calls advance) and resets rows
// logically; it never touches device memory and makes no HIP call.
#include <algorithm>
#include <cstdio>
#include <deque>
#include <set>
#include <unordered_map>
#include <vector>

#include "../../include/mllm.h"
#include "host.h"

namespace {

struct Request {
    int32_t prompt_len = 0, max_new = 0;
    int32_t row = -1;        // -1 while queued
    bool planned = false;    // admitted at an earlier boundary: decodes from now on
    bool stop = false, cancel = false;
};

mllm_status failf(mllm_status st, const char *fmt, long long a = 0, long long b = 0,
                  long long c = 0)
{
    char buf[256];
    snprintf(buf, sizeof buf, fmt, a, b, c);
    return mllm::host_fail(st, buf);
}

}  // namespace

struct mllm_sched {
    mllm_cache *cache = nullptr;
    int32_t slots = 0, capacity = 0, max_seq = 0;
    std::deque<int64_t> queue;                  // queued request ids, first in first out
    std::unordered_map<int64_t, Request> reqs;  // queued and active requests
    std::vector<int64_t> row_req;               // request holding each row, or -1
    std::set<int32_t> free_rows;                // the lowest free row is *begin()
};

extern "C" {

mllm_status mllm_sched_create(mllm_cache *cache, int32_t max_sequence_length, mllm_sched **out)
{
    if (!cache || !out)
        return failf(MLLM_ERR_INVALID_ARG, "cache and out must be non-null");
    mllm_cache_desc d;
    mllm_status st = mllm_cache_get_desc(cache, &d);
    if (st)
        return st;
    if (max_sequence_length < 0 || max_sequence_length > d.capacity)
        return failf(MLLM_ERR_OUT_OF_RANGE,
                     "max_sequence_length %lld outside [0, capacity %lld] (0 = capacity)",
                     max_sequence_length, d.capacity);
    for (int32_t r = 0; r < d.slots; ++r) {
        int32_t len = 0;
        if ((st = mllm_cache_row_length(cache, r, &len)))
            return st;
        if (len != 0)
            return failf(MLLM_ERR_ROW_BUSY,
                         "cache row %lld holds %lld positions: the scheduler owns every row, "
                         "reset them first", r, len);
    }
    mllm_sched *s = new mllm_sched;
    s->cache = cache;
    s->slots = d.slots;
    s->capacity = d.capacity;
    s->max_seq = max_sequence_length ? max_sequence_length : d.capacity;
    s->row_req.assign(d.slots, -1);
    for (int32_t r = 0; r < d.slots; ++r)
        s->free_rows.insert(r);
    *out = s;
    return mllm::host_ok();
}

mllm_status mllm_sched_free(mllm_sched *s)
{
    delete s;
    return mllm::host_ok();
}

mllm_status mllm_sched_max_sequence_length(const mllm_sched *s, int32_t *len)
{
    if (!s || !len)
        return failf(MLLM_ERR_INVALID_ARG, "scheduler and len must be non-null");
    *len = s->max_seq;
    return mllm::host_ok();
}

mllm_status mllm_sched_submit(mllm_sched *s, int64_t request_id, int32_t prompt_len,
                              int32_t max_new_tokens)
{
    if (!s)
        return failf(MLLM_ERR_INVALID_ARG, "scheduler is null");
    if (prompt_len < 1 || max_new_tokens < 0)
        return failf(MLLM_ERR_INVALID_ARG, "need prompt_len >= 1 and max_new_tokens >= 0 "
                     "(got %lld, %lld)", prompt_len, max_new_tokens);
    if ((int64_t)prompt_len + max_new_tokens > s->max_seq)
        return failf(MLLM_ERR_OUT_OF_RANGE, "prompt %lld + new tokens %lld exceed "
                     "max_sequence_length %lld", prompt_len, max_new_tokens, s->max_seq);
    if (s->reqs.count(request_id))
        return failf(MLLM_ERR_INVALID_ARG, "request %lld is already queued or active",
                     request_id);
    Request q;
    q.prompt_len = prompt_len;
    q.max_new = max_new_tokens;
    s->reqs.emplace(request_id, q);
    s->queue.push_back(request_id);
    return mllm::host_ok();
}

static mllm_status mark_end(mllm_sched *s, int64_t request_id, bool cancel)
{
    if (!s)
        return failf(MLLM_ERR_INVALID_ARG, "scheduler is null");
    auto it = s->reqs.find(request_id);
    if (it == s->reqs.end())
        return failf(MLLM_ERR_INVALID_ARG, "request %lld is neither queued nor active",
                     request_id);
    if (cancel && it->second.row < 0) {  // still queued: leaves the queue now
        s->queue.erase(std::find(s->queue.begin(), s->queue.end(), request_id));
        s->reqs.erase(it);
        return mllm::host_ok();
    }
    (cancel ? it->second.cancel : it->second.stop) = true;
    return mllm::host_ok();
}

mllm_status mllm_sched_stop(mllm_sched *s, int64_t request_id)
{
    return mark_end(s, request_id, false);
}

mllm_status mllm_sched_cancel(mllm_sched *s, int64_t request_id)
{
    return mark_end(s, request_id, true);
}

mllm_status mllm_sched_boundary(mllm_sched *s, mllm_sched_entry *admitted, int32_t admitted_cap,
                                int32_t *n_admitted, mllm_sched_entry *decode,
                                int32_t decode_cap, int32_t *n_decode,
                                mllm_sched_entry *retired, int32_t retired_cap,
                                int32_t *n_retired)
{
    if (!s || !n_admitted || !n_decode || !n_retired)
        return failf(MLLM_ERR_INVALID_ARG, "scheduler and the three counts must be non-null");
    if (admitted_cap < s->slots || decode_cap < s->slots || retired_cap < s->slots ||
        !admitted || !decode || !retired)
        return failf(MLLM_ERR_INVALID_ARG, "each plan array needs room for %lld entries "
                     "(the cache's slots)", s->slots);
    // read every active row's length first, so a failure changes nothing
    std::vector<int32_t> len(s->slots, 0);
    for (int32_t r = 0; r < s->slots; ++r) {
        if (s->row_req[r] < 0)
            continue;
        mllm_status st = mllm_cache_row_length(s->cache, r, &len[r]);
        if (st)
            return st;
    }

    // 1. retire: length reached, stopped or cancelled; the row is reset and freed
    int32_t nr = 0;
    for (int32_t r = 0; r < s->slots; ++r) {
        const int64_t id = s->row_req[r];
        if (id < 0)
            continue;
        const Request &q = s->reqs.at(id);
        int32_t why = 0;
        if (q.cancel)
            why = MLLM_END_CANCEL;
        else if (q.stop)
            why = MLLM_END_STOP;
        else if (q.planned && len[r] >= q.prompt_len + q.max_new)
            why = MLLM_END_LENGTH;
        if (!why)
            continue;
        mllm_status st = mllm_cache_reset_row(s->cache, r);
        if (st)
            return st;
        retired[nr++] = mllm_sched_entry{id, r, why};
        s->row_req[r] = -1;
        s->free_rows.insert(r);
        s->reqs.erase(id);
    }

    // 2. decode: the requests admitted at an earlier boundary, by row, at the
    //    position their next token goes to
    int32_t nd = 0;
    for (int32_t r = 0; r < s->slots; ++r) {
        const int64_t id = s->row_req[r];
        if (id >= 0 && s->reqs.at(id).planned)
            decode[nd++] = mllm_sched_entry{id, r, len[r]};
    }

    // 3. admit: first in first out into the lowest free rows
    int32_t na = 0;
    while (!s->queue.empty() && !s->free_rows.empty()) {
        const int64_t id = s->queue.front();
        s->queue.pop_front();
        const int32_t r = *s->free_rows.begin();
        s->free_rows.erase(s->free_rows.begin());
        Request &q = s->reqs.at(id);
        q.row = r;
        s->row_req[r] = id;
        admitted[na++] = mllm_sched_entry{id, r, q.prompt_len};
    }
    // equal prompt lengths next to each other (one prefill group each), by row within
    std::stable_sort(admitted, admitted + na, [](const mllm_sched_entry &x, const mllm_sched_entry &y) {
        return x.value != y.value ? x.value < y.value : x.row < y.row;
    });
    // requests admitted now decode from the next boundary on
    for (int32_t i = 0; i < na; ++i)
        s->reqs.at(admitted[i].request_id).planned = true;
    *n_admitted = na;
    *n_decode = nd;
    *n_retired = nr;
    return mllm::host_ok();
}

mllm_status mllm_sched_counts(const mllm_sched *s, int32_t *queued, int32_t *active)
{
    if (!s || !queued || !active)
        return failf(MLLM_ERR_INVALID_ARG, "scheduler and counts must be non-null");
    *queued = (int32_t)s->queue.size();
    *active = (int32_t)(s->reqs.size() - s->queue.size());
    return mllm::host_ok();
}

}  // extern "C"
