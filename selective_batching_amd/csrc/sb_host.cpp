// Host half of libsb: error reporting, the K/V manager, the iteration-level
// scheduler and the ragged-batch metadata / attention work-list builder.
//
// Sources: Algorithm 1 (Select) and its notes in "连续批处理完全拆解"
// (sections 迭代级 FCFS, 两个约束, Figure 5 K/V manager); sections 4.1-4.3 and
// 5.1 of "CS349D Lecture 2 · 批处理与调度"; select_batch in "Orca: The
// beginning of Morden LLM serving" (Scheduling Algorithm).
#include <algorithm>
#include <climits>
#include <array>
#include <cstdio>
#include <cstring>
#include <memory>

#include "sb_internal.h"

namespace {
thread_local std::string g_err;
}

namespace sb {

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int validate_dims(const sb_model_dims* d) {
    if (!d) return fail(SB_ERR_INVALID, "dims is NULL");
    if (d->arch != SB_ARCH_GPT && d->arch != SB_ARCH_LLAMA) return fail(SB_ERR_INVALID, "unknown arch %d", d->arch);
    if (d->dtype != SB_F32 && d->dtype != SB_BF16) return fail(SB_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->hidden <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0)
        return fail(SB_ERR_INVALID, "non-positive model dimension");
    if (d->n_heads % d->n_kv_heads) return fail(SB_ERR_INVALID, "n_heads %% n_kv_heads != 0");
    int g = d->n_heads / d->n_kv_heads;
    if (kRowsPerWave % g) return fail(SB_ERR_INVALID, "query heads per K/V head (%d) must divide 16", g);
    if (d->hidden % 64 || d->ffn % 64 || (d->n_heads * d->head_dim) % 64)
        return fail(SB_ERR_INVALID, "hidden, ffn and n_heads*head_dim must be multiples of 64");
    // exactly the head dims the attention kernel is instantiated for
    const int hd = d->head_dim;
    if (d->dtype == SB_BF16 && hd != 32 && hd != 64 && hd != 128)
        return fail(SB_ERR_INVALID, "bf16 head_dim must be 32, 64 or 128 (got %d)", hd);
    if (d->dtype == SB_F32 && hd != 16 && hd != 32 && hd != 64 && hd != 128)
        return fail(SB_ERR_INVALID, "fp32 head_dim must be 16, 32, 64 or 128 (got %d)", hd);
    if (d->arch == SB_ARCH_LLAMA && d->head_dim % 2) return fail(SB_ERR_INVALID, "RoPE needs an even head_dim");
    return SB_OK;
}

}  // namespace sb

using sb::fail;

extern "C" const char* sb_last_error(void) { return g_err.c_str(); }

// ============================================================== K/V manager

extern "C" int64_t sb_kv_arena_slots(int64_t n_slots, int32_t max_live) {
    if (n_slots < 0 || max_live < 0) return -1;
    return sb::round_up(n_slots, 8) + 8 * (int64_t)max_live;
}

extern "C" size_t sb_kv_arena_bytes(int64_t arena_slots, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t dtype) {
    if (arena_slots < 0 || n_layers <= 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
    return (size_t)arena_slots * n_layers * n_kv_heads * head_dim * sb::dtype_size(dtype);
}

extern "C" int sb_kv_create(int64_t n_slots, int64_t arena_slots, int32_t n_layers, int32_t n_kv_heads,
                            int32_t head_dim, int32_t dtype, void* k_arena, void* v_arena, sb_kv** out) {
    if (!out) return fail(SB_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (n_slots <= 0 || n_layers <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return fail(SB_ERR_INVALID, "non-positive K/V manager size");
    if (dtype != SB_F32 && dtype != SB_BF16) return fail(SB_ERR_INVALID, "unknown dtype %d", dtype);
    if (arena_slots < n_slots || arena_slots % 8)
        return fail(SB_ERR_INVALID, "arena_slots (%lld) must be a multiple of 8 and >= n_slots (%lld)",
                    (long long)arena_slots, (long long)n_slots);
    if (arena_slots >= (int64_t(1) << 31)) return fail(SB_ERR_INVALID, "arena_slots must be < 2^31");
    if ((k_arena == nullptr) != (v_arena == nullptr)) return fail(SB_ERR_INVALID, "give both arenas or neither");
    auto* kv = new sb_kv();
    kv->n_slots = n_slots;
    kv->arena_slots = arena_slots;
    kv->n_layers = n_layers;
    kv->nkv = n_kv_heads;
    kv->d = head_dim;
    kv->dtype = dtype;
    kv->k = k_arena;
    kv->v = v_arena;
    *out = kv;
    return SB_OK;
}

extern "C" int sb_kv_set_stream(sb_kv* kv, void* stream) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    kv->stream = (hipStream_t)stream;
    return SB_OK;
}

namespace {

// Copy one live range left (dst < src) in every (layer, kv head) plane of
// both arenas.  Chunks never longer than the shift keep each chunk's source
// and destination apart; ascending chunk order never overwrites a source
// that is still to be read.  All offsets are multiples of 8 slots, so the
// blocked V layout moves with the same byte arithmetic as K.
int move_range(sb_kv* kv, int64_t src, int64_t dst, int64_t len) {
    if (!kv->k || src == dst || len == 0) return SB_OK;
    const size_t es = sb::dtype_size(kv->dtype);
    const size_t row = (size_t)kv->d * es;
    const size_t pitch = (size_t)kv->arena_slots * row;
    const size_t planes = (size_t)kv->n_layers * kv->nkv;
    const int64_t chunk = std::min<int64_t>(len, src - dst);
    for (int64_t off = 0; off < len; off += chunk) {
        int64_t c = std::min<int64_t>(chunk, len - off);
        for (void* base : {kv->k, kv->v}) {
            char* b = (char*)base;
            hipError_t e = hipMemcpy2DAsync(b + (dst + off) * row, pitch, b + (src + off) * row, pitch,
                                            (size_t)c * row, planes, hipMemcpyDeviceToDevice, kv->stream);
            if (e != hipSuccess) return fail(SB_ERR_DEVICE, "K/V compaction copy: %s", hipGetErrorString(e));
        }
    }
    return SB_OK;
}

// First-fit placement of len slots; returns -1 when no hole is large enough.
int64_t first_fit(const sb_kv* kv, int64_t len) {
    int64_t end = 0;
    for (const auto& [base, id] : kv->by_base) {
        if (base - end >= len) return end;
        end = base + kv->live.at(id).len;
    }
    return kv->arena_slots - end >= len ? end : -1;
}

int compact(sb_kv* kv) {
    std::map<int64_t, int64_t> packed;
    int64_t end = 0;
    for (const auto& [base, id] : kv->by_base) {
        auto& r = kv->live.at(id);
        if (base != end) {
            int st = move_range(kv, base, end, r.len);
            if (st) return st;
            r.base = end;
        }
        packed[end] = id;
        end += r.len;
    }
    kv->by_base.swap(packed);
    kv->n_compactions++;
    return SB_OK;
}

}  // namespace

extern "C" int sb_kv_reserve(sb_kv* kv, int64_t req_id, int32_t max_tokens, int64_t* slot_base) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    if (max_tokens <= 0) return fail(SB_ERR_INVALID, "max_tokens must be positive");
    if (kv->live.count(req_id)) return fail(SB_ERR_STATE, "request %lld already holds a reservation", (long long)req_id);
    if (max_tokens > kv->n_slots) return fail(SB_ERR_TOO_LARGE, "max_tokens %d > n_slots %lld", max_tokens, (long long)kv->n_slots);
    // Admission is decided by the counter alone: fail iff n_rsrv + max_tokens > n_slots.
    if (kv->n_rsrv + max_tokens > kv->n_slots)
        return fail(SB_ERR_NO_SLOTS, "n_rsrv %lld + %d > n_slots %lld", (long long)kv->n_rsrv, max_tokens, (long long)kv->n_slots);
    const int64_t len = sb::round_up(max_tokens, 8);
    int64_t base = first_fit(kv, len);
    if (base < 0) {
        int st = compact(kv);
        if (st) return st;
        base = first_fit(kv, len);
        if (base < 0)
            return fail(SB_ERR_CAPACITY, "arena of %lld slots cannot place %lld more after compaction; size it with sb_kv_arena_slots",
                        (long long)kv->arena_slots, (long long)len);
    }
    kv->live[req_id] = {base, len, max_tokens};
    kv->by_base[base] = req_id;
    kv->n_rsrv += max_tokens;
    if (slot_base) *slot_base = base;
    return SB_OK;
}

extern "C" int sb_kv_free(sb_kv* kv, int64_t req_id) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    auto it = kv->live.find(req_id);
    if (it == kv->live.end()) return fail(SB_ERR_NOT_FOUND, "request %lld holds no reservation", (long long)req_id);
    kv->n_rsrv -= it->second.max_tokens;
    kv->by_base.erase(it->second.base);
    kv->live.erase(it);
    return SB_OK;
}

extern "C" int sb_kv_lookup(const sb_kv* kv, int64_t req_id, int64_t* slot_base, int32_t* max_tokens) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    auto it = kv->live.find(req_id);
    if (it == kv->live.end()) return fail(SB_ERR_NOT_FOUND, "request %lld holds no reservation", (long long)req_id);
    if (slot_base) *slot_base = it->second.base;
    if (max_tokens) *max_tokens = it->second.max_tokens;
    return SB_OK;
}

extern "C" int sb_kv_stats(const sb_kv* kv, int64_t* n_rsrv, int64_t* n_slots, int64_t* n_live, int64_t* n_compactions) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    if (n_rsrv) *n_rsrv = kv->n_rsrv;
    if (n_slots) *n_slots = kv->n_slots;
    if (n_live) *n_live = (int64_t)kv->live.size();
    if (n_compactions) *n_compactions = kv->n_compactions;
    return SB_OK;
}

extern "C" int sb_kv_layer_ptrs(const sb_kv* kv, int32_t layer, void** k, void** v) {
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    if (layer < 0 || layer >= kv->n_layers) return fail(SB_ERR_INVALID, "layer %d out of range", layer);
    if (!kv->k) return fail(SB_ERR_STATE, "K/V manager has no device arenas");
    size_t plane = (size_t)kv->nkv * kv->arena_slots * kv->d * sb::dtype_size(kv->dtype);
    if (k) *k = (char*)kv->k + plane * layer;
    if (v) *v = (char*)kv->v + plane * layer;
    return SB_OK;
}

extern "C" void sb_kv_destroy(sb_kv* kv) { delete kv; }

// ============================================================== scheduler

namespace {
enum { ST_INITIATION = 0, ST_RUNNING = 1, ST_INCREMENT = 2 };

struct Req {
    int64_t id;
    double arrival;
    int64_t order;
    int32_t prompt_len, out_len, max_tokens;
    int32_t state;
    int32_t generated;
    std::vector<int32_t> prompt;
    std::vector<int32_t> out;
    int32_t prefilled = 0;                          // prompt tokens already processed (K/V cached)
    int32_t cur_new = 0;                            // tokens fed in the current iteration
    int64_t pending_ticket = -1;                    // deferred completion whose token value is not known yet
    int32_t pending_row = -1;                       // this request's row in that iteration's batch
};
}  // namespace

struct sb_sched {
    int32_t max_bs = 0;
    sb_kv* kv = nullptr;
    std::vector<Req*> pool;                         // kept sorted by (arrival, order)
    std::unordered_map<int64_t, std::unique_ptr<Req>> by_id;
    std::unordered_map<int64_t, std::vector<int32_t>> done;
    int64_t next_order = 0;
    int64_t n_finished = 0;
    int32_t budget = 0, chunk = 0;                  // chunked prefill (0: whole prompts, Algorithm 1)
    bool request_level = false;                     // static batching: whole batches start and end together
    std::vector<Req*> seated;                       // its running batch's unfinished members (batch order)
    // deferred completions: ticket -> (request id, position of the pending token in its output), batch order
    std::map<int64_t, std::vector<std::pair<int64_t, int32_t>>> tickets;
    int64_t next_ticket = 0;
};

extern "C" int sb_sched_create(int32_t max_bs, sb_kv* kv, sb_sched** out) {
    if (!out) return fail(SB_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (max_bs <= 0) return fail(SB_ERR_INVALID, "max_bs must be positive (got %d)", max_bs);
    if (!kv) return fail(SB_ERR_INVALID, "kv is NULL");
    auto* s = new sb_sched();
    s->max_bs = max_bs;
    s->kv = kv;
    *out = s;
    return SB_OK;
}

namespace {
int insert_req(sb_sched* s, std::unique_ptr<Req> r) {
    Req* p = r.get();
    auto pos = std::upper_bound(s->pool.begin(), s->pool.end(), p, [](const Req* a, const Req* b) {
        return a->arrival < b->arrival || (a->arrival == b->arrival && a->order < b->order);
    });
    s->pool.insert(pos, p);
    s->by_id[p->id] = std::move(r);
    return SB_OK;
}

int check_new(sb_sched* s, int64_t req_id, int32_t prompt_len, int32_t out_len, int32_t max_tokens) {
    if (!s) return fail(SB_ERR_INVALID, "sched is NULL");
    if (s->by_id.count(req_id) || s->done.count(req_id))
        return fail(SB_ERR_STATE, "request id %lld already submitted", (long long)req_id);
    if (prompt_len < 1 || out_len < 1 || max_tokens < 1) return fail(SB_ERR_INVALID, "lengths must be >= 1");
    if (max_tokens > s->kv->n_slots)
        return fail(SB_ERR_TOO_LARGE, "request %lld: max_tokens %d > n_slots %lld", (long long)req_id, max_tokens,
                    (long long)s->kv->n_slots);
    // the last iteration writes slot prompt_len + out_len - 2: the history must fit the reservation
    if ((int64_t)prompt_len + out_len - 1 > max_tokens)
        return fail(SB_ERR_INVALID, "request %lld: prompt_len + out_len - 1 > max_tokens", (long long)req_id);
    return SB_OK;
}
}  // namespace

extern "C" int sb_sched_add(sb_sched* s, int64_t req_id, double arrival, int32_t prompt_len,
                            const int32_t* prompt_tokens, int32_t out_len, int32_t max_tokens) {
    int st = check_new(s, req_id, prompt_len, out_len, max_tokens);
    if (st) return st;
    auto r = std::make_unique<Req>();
    r->id = req_id;
    r->arrival = arrival;
    r->order = s->next_order++;
    r->prompt_len = prompt_len;
    r->out_len = out_len;
    r->max_tokens = max_tokens;
    r->state = ST_INITIATION;
    r->generated = 0;
    r->prompt.assign(prompt_len, 0);
    if (prompt_tokens) std::memcpy(r->prompt.data(), prompt_tokens, sizeof(int32_t) * prompt_len);
    return insert_req(s, std::move(r));
}

extern "C" int sb_sched_add_running(sb_sched* s, int64_t req_id, double arrival, int32_t prompt_len,
                                    const int32_t* prompt_tokens, int32_t out_len, int32_t max_tokens,
                                    int32_t generated, int32_t last_token) {
    int st = check_new(s, req_id, prompt_len, out_len, max_tokens);
    if (st) return st;
    if (generated < 1 || generated >= out_len)
        return fail(SB_ERR_INVALID, "generated must be in [1, out_len)");
    st = sb_kv_reserve(s->kv, req_id, max_tokens, nullptr);
    if (st) return st;
    auto r = std::make_unique<Req>();
    r->id = req_id;
    r->arrival = arrival;
    r->order = s->next_order++;
    r->prompt_len = prompt_len;
    r->out_len = out_len;
    r->max_tokens = max_tokens;
    r->state = ST_INCREMENT;
    r->generated = generated;
    r->prefilled = prompt_len;
    r->prompt.assign(prompt_len, 0);
    if (prompt_tokens) std::memcpy(r->prompt.data(), prompt_tokens, sizeof(int32_t) * prompt_len);
    r->out.assign(generated, 0);
    r->out.back() = last_token;
    return insert_req(s, std::move(r));
}

extern "C" int sb_sched_set_request_level(sb_sched* s, int32_t on) {
    if (!s) return fail(SB_ERR_INVALID, "sched is NULL");
    if (on && s->budget) return fail(SB_ERR_INVALID, "request-level batching feeds whole prompts (chunking is on)");
    if (!on) s->seated.clear();
    s->request_level = on != 0;
    return SB_OK;
}

extern "C" int sb_sched_set_chunking(sb_sched* s, int32_t token_budget, int32_t chunk) {
    if (!s) return fail(SB_ERR_INVALID, "sched is NULL");
    if (token_budget && s->request_level) return fail(SB_ERR_INVALID, "chunking needs iteration-level scheduling");
    if (token_budget < 0 || chunk < 0 || (token_budget == 0) != (chunk == 0))
        return fail(SB_ERR_INVALID, "token_budget and chunk: both positive, or both 0 (off)");
    s->budget = token_budget;
    s->chunk = chunk;
    return SB_OK;
}

extern "C" int sb_select_batch(sb_sched* s, int32_t cap, int64_t* ids, int32_t* n_new, int32_t* ctx,
                               int64_t* slot_base, int32_t* n_out) {
    if (!s || !n_out) return fail(SB_ERR_INVALID, "NULL argument");
    *n_out = 0;
    if (cap < std::min<int64_t>(s->max_bs, (int64_t)s->pool.size()))
        return fail(SB_ERR_CAPACITY, "cap %d < min(max_bs, pool size)", cap);
    std::vector<std::pair<Req*, int32_t>> batch;    // member, tokens it feeds this iteration
    auto admit = [&](Req* r, int* st) {             // first scheduling: reserve max_tokens (stop on failure)
        *st = SB_OK;
        if (r->state != ST_INITIATION) return true;
        *st = sb_kv_reserve(s->kv, r->id, r->max_tokens, nullptr);
        if (*st == SB_ERR_NO_SLOTS) {
            *st = SB_OK;
            return false;
        }
        return *st == SB_OK;
    };
    int st = SB_OK;
    if (s->request_level && !s->seated.empty()) {
        for (Req* r : s->seated) batch.push_back({r, 1}); // the running batch continues, nobody joins
    } else if (s->budget == 0) {
        for (Req* r : s->pool) {                          // arrival order
            if (r->state == ST_RUNNING) continue;
            if ((int32_t)batch.size() == s->max_bs) break;
            if (!admit(r, &st)) break;                    // stop, never skip: FCFS
            batch.push_back({r, r->prefilled < r->prompt_len ? r->prompt_len - r->prefilled : 1});
        }
    } else {
        int64_t left = s->budget;
        for (Req* r : s->pool) {                          // decodes first, one token each
            if (r->state == ST_RUNNING || r->prefilled < r->prompt_len) continue;
            if ((int32_t)batch.size() == s->max_bs || left == 0) break;
            batch.push_back({r, 1});
            left -= 1;
        }
        for (Req* r : s->pool) {                          // then prompt chunks, arrival order
            if (r->state == ST_RUNNING || r->prefilled == r->prompt_len) continue;
            if ((int32_t)batch.size() == s->max_bs || left == 0) break;
            if (!admit(r, &st)) break;
            const int32_t n = (int32_t)std::min<int64_t>({(int64_t)s->chunk, (int64_t)(r->prompt_len - r->prefilled), left});
            batch.push_back({r, n});
            left -= n;
        }
    }
    if (st) return st;
    if (s->request_level && s->seated.empty())
        for (auto& b : batch) s->seated.push_back(b.first);
    for (size_t i = 0; i < batch.size(); ++i) {
        Req* r = batch[i].first;
        r->state = ST_RUNNING;
        r->cur_new = batch[i].second;
        if (ids) ids[i] = r->id;
        const bool prompt = r->prefilled < r->prompt_len;
        if (n_new) n_new[i] = r->cur_new;
        if (ctx) ctx[i] = prompt ? r->prefilled : r->prompt_len + r->generated - 1;
        // The manager's base, read after the whole batch is admitted: a later member's reservation may
        // have compacted the arena and moved the ranges of members admitted before it.
        if (slot_base) slot_base[i] = s->kv->live.at(r->id).base;
    }
    *n_out = (int32_t)batch.size();
    return SB_OK;
}

extern "C" int sb_batch_tokens(const sb_sched* s, int32_t n, const int64_t* ids, int32_t cap, int32_t* tokens,
                               int32_t* n_tokens) {
    if (!s || (n > 0 && !ids) || !n_tokens) return fail(SB_ERR_INVALID, "NULL argument");
    int32_t t = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->by_id.find(ids[i]);
        if (it == s->by_id.end()) return fail(SB_ERR_NOT_FOUND, "request %lld not in the pool", (long long)ids[i]);
        const Req* r = it->second.get();
        if (r->state != ST_RUNNING) return fail(SB_ERR_STATE, "request %lld is not in the running batch", (long long)ids[i]);
        if (r->prefilled < r->prompt_len) {                 // (a chunk of) the prompt
            if (t + r->cur_new > cap) return fail(SB_ERR_CAPACITY, "token capacity %d exceeded", cap);
            if (tokens) std::memcpy(tokens + t, r->prompt.data() + r->prefilled, sizeof(int32_t) * r->cur_new);
            t += r->cur_new;
        } else {
            if (t + 1 > cap) return fail(SB_ERR_CAPACITY, "token capacity %d exceeded", cap);
            if (r->pending_ticket >= 0)
                return fail(SB_ERR_STATE, "request %lld: its last token is still pending (use sb_batch_token_refs)",
                            (long long)ids[i]);
            if (tokens) tokens[t] = r->out.back();
            t += 1;
        }
    }
    *n_tokens = t;
    return SB_OK;
}

extern "C" int sb_batch_token_refs(const sb_sched* s, int32_t n, const int64_t* ids, int32_t cap, int32_t* tokens,
                                   int32_t* n_tokens, int64_t* ref_ticket) {
    if (!s || (n > 0 && !ids) || !n_tokens || !ref_ticket) return fail(SB_ERR_INVALID, "NULL argument");
    int32_t t = 0;
    int64_t ticket = -1;
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->by_id.find(ids[i]);
        if (it == s->by_id.end()) return fail(SB_ERR_NOT_FOUND, "request %lld not in the pool", (long long)ids[i]);
        const Req* r = it->second.get();
        if (r->state != ST_RUNNING) return fail(SB_ERR_STATE, "request %lld is not in the running batch", (long long)ids[i]);
        if (r->prefilled < r->prompt_len) {                 // (a chunk of) the prompt
            if (t + r->cur_new > cap) return fail(SB_ERR_CAPACITY, "token capacity %d exceeded", cap);
            if (tokens) std::memcpy(tokens + t, r->prompt.data() + r->prefilled, sizeof(int32_t) * r->cur_new);
            t += r->cur_new;
        } else {
            if (t + 1 > cap) return fail(SB_ERR_CAPACITY, "token capacity %d exceeded", cap);
            int32_t v = r->out.back();
            if (r->pending_ticket >= 0) {
                if (ticket >= 0 && ticket != r->pending_ticket)
                    return fail(SB_ERR_STATE, "pending tokens of the batch come from more than one iteration");
                ticket = r->pending_ticket;
                v = -1 - r->pending_row;
            }
            if (tokens) tokens[t] = v;
            t += 1;
        }
    }
    *n_tokens = t;
    *ref_ticket = ticket;
    return SB_OK;
}

namespace {
// Complete of Algorithm 1: every member generated one token (value new_tokens[i], or pending under
// `ticket` when new_tokens is NULL and ticket >= 0); members that reached out_len finish and free slots.
int complete_batch(sb_sched* s, int32_t n, const int64_t* ids, const int32_t* new_tokens, int64_t ticket,
                   int32_t* n_finished, int64_t* finished_ids) {
    if (!s || (n > 0 && !ids)) return fail(SB_ERR_INVALID, "NULL argument");
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->by_id.find(ids[i]);
        if (it == s->by_id.end()) return fail(SB_ERR_NOT_FOUND, "request %lld not in the pool", (long long)ids[i]);
        if (it->second->state != ST_RUNNING) return fail(SB_ERR_STATE, "request %lld did not run", (long long)ids[i]);
    }
    int32_t nf = 0;
    std::vector<std::pair<int64_t, int32_t>> slots_of_ticket;
    for (int32_t i = 0; i < n; ++i) {
        Req* r = s->by_id.at(ids[i]).get();
        r->state = ST_INCREMENT;
        if (r->prefilled < r->prompt_len) {
            r->prefilled += r->cur_new;
            if (r->prefilled < r->prompt_len) {              // a chunk short of the prompt's end: no token
                if (ticket >= 0) slots_of_ticket.push_back({r->id, -1});
                continue;
            }
        }
        if (ticket >= 0) {
            slots_of_ticket.push_back({r->id, (int32_t)r->out.size()});
            r->pending_ticket = ticket;
            r->pending_row = i;
        }
        r->out.push_back(new_tokens ? new_tokens[i] : 0);
        r->generated += 1;
        if (r->generated == r->out_len) {
            int st = sb_kv_free(s->kv, r->id);
            if (st) return st;
            if (finished_ids) finished_ids[nf] = r->id;
            nf++;
            s->n_finished++;
            s->pool.erase(std::find(s->pool.begin(), s->pool.end(), r));
            auto seat = std::find(s->seated.begin(), s->seated.end(), r);
            if (seat != s->seated.end()) s->seated.erase(seat);
            s->done[r->id] = std::move(r->out);
            s->by_id.erase(r->id);
        }
    }
    if (ticket >= 0) s->tickets[ticket] = std::move(slots_of_ticket);
    if (n_finished) *n_finished = nf;
    return SB_OK;
}
}  // namespace

extern "C" int sb_sched_complete(sb_sched* s, int32_t n, const int64_t* ids, const int32_t* new_tokens,
                                 int32_t* n_finished, int64_t* finished_ids) {
    return complete_batch(s, n, ids, new_tokens, -1, n_finished, finished_ids);
}

extern "C" int sb_sched_complete_deferred(sb_sched* s, int32_t n, const int64_t* ids, int32_t* n_finished,
                                          int64_t* finished_ids, int64_t* ticket) {
    if (!s || !ticket) return fail(SB_ERR_INVALID, "NULL argument");
    const int64_t tk = s->next_ticket;
    int st = complete_batch(s, n, ids, nullptr, tk, n_finished, finished_ids);
    if (st) return st;
    s->next_ticket++;
    *ticket = tk;
    return SB_OK;
}

extern "C" int sb_sched_set_tokens(sb_sched* s, int64_t ticket, int32_t n, const int32_t* tokens) {
    if (!s || (n > 0 && !tokens)) return fail(SB_ERR_INVALID, "NULL argument");
    auto t = s->tickets.find(ticket);
    if (t == s->tickets.end()) return fail(SB_ERR_NOT_FOUND, "unknown or already settled ticket %lld", (long long)ticket);
    if ((int32_t)t->second.size() != n)
        return fail(SB_ERR_INVALID, "ticket %lld covers %zu requests, %d tokens given", (long long)ticket,
                    t->second.size(), n);
    for (int32_t i = 0; i < n; ++i) {
        const int64_t id = t->second[i].first;
        const int32_t pos = t->second[i].second;
        if (pos < 0) continue;                               // that member yielded no token
        auto live = s->by_id.find(id);
        if (live != s->by_id.end()) {
            Req* r = live->second.get();
            r->out[pos] = tokens[i];
            if (r->pending_ticket == ticket) {
                r->pending_ticket = -1;
                r->pending_row = -1;
            }
        } else {
            s->done.at(id)[pos] = tokens[i];
        }
    }
    s->tickets.erase(t);
    return SB_OK;
}

extern "C" int sb_sched_output(const sb_sched* s, int64_t req_id, int32_t cap, int32_t* tokens, int32_t* n) {
    if (!s || !n) return fail(SB_ERR_INVALID, "NULL argument");
    const std::vector<int32_t>* v = nullptr;
    auto d = s->done.find(req_id);
    if (d != s->done.end()) {
        v = &d->second;
    } else {
        auto it = s->by_id.find(req_id);
        if (it == s->by_id.end()) return fail(SB_ERR_NOT_FOUND, "unknown request %lld", (long long)req_id);
        v = &it->second->out;
    }
    *n = (int32_t)v->size();
    if ((int32_t)v->size() > cap) return fail(SB_ERR_CAPACITY, "capacity %d < %zu tokens", cap, v->size());
    if (tokens && !v->empty()) std::memcpy(tokens, v->data(), sizeof(int32_t) * v->size());
    return SB_OK;
}

extern "C" int sb_reservation_tokens(int32_t policy, int32_t prompt_len, int32_t out_len, int32_t max_out,
                                     int32_t* max_tokens) {
    if (!max_tokens) return fail(SB_ERR_INVALID, "NULL argument");
    if (prompt_len < 1 || out_len < 1 || out_len > max_out || max_out > (1 << 30))
        return fail(SB_ERR_INVALID, "need 1 <= out_len <= max_out <= 2^30 and prompt_len >= 1");
    int64_t v;
    switch (policy) {
        case SB_RESERVE_MAX: v = (int64_t)prompt_len + max_out; break;
        case SB_RESERVE_POW2: {
            int64_t p = 1;
            while (p < out_len) p *= 2;
            v = (int64_t)prompt_len + p;
            break;
        }
        case SB_RESERVE_ORACLE: v = (int64_t)prompt_len + out_len - 1; break;
        default: return fail(SB_ERR_INVALID, "unknown reservation policy %d", policy);
    }
    if (v > INT32_MAX) return fail(SB_ERR_INVALID, "reservation overflows int32");
    *max_tokens = (int32_t)v;
    return SB_OK;
}

extern "C" int sb_kv_usage(const sb_sched* s, int64_t* reserved, int64_t* stored) {
    if (!s || !reserved || !stored) return fail(SB_ERR_INVALID, "NULL argument");
    int64_t st = 0;
    for (const Req* r : s->pool) {
        if (r->state == ST_RUNNING)                  // this iteration's tokens counted as written
            st += (r->prefilled < r->prompt_len ? r->prefilled : (int64_t)r->prompt_len + r->generated - 1) + r->cur_new;
        else
            st += r->prefilled + std::max(r->generated - 1, 0);
    }
    *reserved = s->kv->n_rsrv;
    *stored = st;
    return SB_OK;
}

extern "C" int sb_sched_stats(const sb_sched* s, int32_t* pool_size, int64_t* n_rsrv, int64_t* n_finished) {
    if (!s) return fail(SB_ERR_INVALID, "sched is NULL");
    if (pool_size) *pool_size = (int32_t)s->pool.size();
    if (n_rsrv) *n_rsrv = s->kv->n_rsrv;
    if (n_finished) *n_finished = s->n_finished;
    return SB_OK;
}

extern "C" void sb_sched_destroy(sb_sched* s) { delete s; }

// ============================================================== ragged metadata

namespace {
constexpr int32_t kMaxTokenRef = 1 << 20;            // token references -(1 + j), j < 2^20
struct Layout {
    size_t cu, ctx, last, pos, slot, ids, items, groups, total;  // int32 offsets
};

Layout layout_for(int64_t B, int64_t T, int64_t n_items, int64_t n_groups) {
    Layout L{};
    size_t o = 0;
    auto take = [&](int64_t n) { size_t r = o; o += (size_t)sb::round_up(n, 16); return r; };
    L.cu = take(B + 1);
    L.ctx = take(B);
    L.last = take(B);
    L.pos = take(T);
    L.slot = take(T);
    L.ids = take(T);
    L.items = take(n_items * sb::kItemInts);
    L.groups = take(n_groups * sb::kGroupInts);
    L.total = o;
    return L;
}

// Row tiles: per (request, K/V head) ceil(rows / 64) <= rows / 64 + 1; runs: at most one per unit.
constexpr int kXcds = 8;                  // XCDs of an MI355X; workgroups are dealt to them round-robin
constexpr int64_t kItemStartCost = 256;   // start-up of a work item, in keys, for the dispatch order

// Work items of a batch, empty padding items (at most a quarter of the others, plus kXcds) included.
int64_t max_items_bound(const sb_model_dims* d, int64_t B, int64_t T, int64_t keys) {
    const int64_t g = d->n_heads / d->n_kv_heads, nkv = d->n_kv_heads;
    const int64_t n = nkv * ((T * g) / sb::kRowsPerTile + B) + sb::max_units_bound(nkv, B, keys);
    return n + n / 4 + kXcds;
}
}  // namespace

extern "C" size_t sb_ragged_bytes(const sb_model_dims* dims, int32_t max_req, int32_t max_tokens, int64_t max_keys_total) {
    if (sb::validate_dims(dims) || max_req < 0 || max_tokens < 0 || max_keys_total < 0) return 0;
    const int64_t items = max_items_bound(dims, max_req, max_tokens, max_keys_total);
    const int64_t groups = (int64_t)dims->n_kv_heads * max_req;
    return layout_for(max_req, max_tokens, items, groups).total * sizeof(int32_t);
}

extern "C" int64_t sb_attn_max_partials(const sb_model_dims* dims, int32_t max_req, int64_t max_keys_total) {
    if (sb::validate_dims(dims) || max_req < 0 || max_keys_total < 0) return 0;
    return sb::max_units_bound(dims->n_kv_heads, max_req, max_keys_total);
}

extern "C" int sb_ragged_build(const sb_model_dims* dims, int32_t n_req, const int32_t* n_new, const int32_t* ctx,
                               const int64_t* slot_base, const int32_t* token_ids, void* host_staging,
                               void* dev_meta, size_t bytes, void* stream, sb_ragged* out) {
    int st = sb::validate_dims(dims);
    if (st) return st;
    if (!out || n_req < 0 || (n_req > 0 && (!n_new || !ctx || !slot_base)) || !host_staging)
        return fail(SB_ERR_INVALID, "NULL argument");
    const int32_t G = dims->n_heads / dims->n_kv_heads;
    const int32_t nkv = dims->n_kv_heads;
    int64_t T = 0, keys = 0;
    int32_t max_new = 0;
    if (token_ids) {
        int64_t nt = 0;
        for (int32_t i = 0; i < n_req; ++i) nt += n_new[i] > 0 ? n_new[i] : 0;
        for (int64_t t = 0; t < nt; ++t)
            if (token_ids[t] < -kMaxTokenRef || (dims->vocab > 0 && token_ids[t] >= dims->vocab))
                return fail(SB_ERR_INVALID, "token %lld: id %d outside [-%d, vocab)", (long long)t, token_ids[t],
                            kMaxTokenRef);
    }
    for (int32_t i = 0; i < n_req; ++i) {
        if (n_new[i] < 1 || ctx[i] < 0) return fail(SB_ERR_INVALID, "request %d: n_new must be >= 1 and ctx >= 0", i);
        if (slot_base[i] < 0 || slot_base[i] % 8) return fail(SB_ERR_INVALID, "request %d: slot_base must be a non-negative multiple of 8", i);
        if (slot_base[i] + ctx[i] + n_new[i] >= (int64_t(1) << 31)) return fail(SB_ERR_INVALID, "slot index overflows int32");
        if (dims->arch == SB_ARCH_GPT && dims->max_pos > 0 && ctx[i] + n_new[i] > dims->max_pos)
            return fail(SB_ERR_INVALID, "request %d: position %d beyond max_pos %d", i, ctx[i] + n_new[i] - 1, dims->max_pos);
        T += n_new[i];
        keys += (int64_t)ctx[i] + n_new[i];
        max_new = std::max(max_new, n_new[i]);
    }
    if (T >= (int64_t(1) << 31)) return fail(SB_ERR_INVALID, "too many tokens");

    // ---- attention work list (Split as offsets: each item names its request's rows and key range)
    struct Item { int32_t v[sb::kItemInts]; int64_t cost, lane_cost; int32_t grp; };
    std::vector<Item> items;
    std::vector<std::array<int32_t, sb::kGroupInts>> groups;
    // units of the single-tile (request, K/V head) pairs, to size the runs
    int64_t n_units = 0;
    for (int32_t i = 0; i < n_req; ++i)
        if (n_new[i] * G <= sb::kRowsPerWave)
            n_units += (int64_t)nkv * ((ctx[i] + n_new[i] + sb::kUnitKeys - 1) / sb::kUnitKeys);
    // units per run: about kTargetRuns runs per launch -- long runs keep a workgroup streaming one
    // request's keys, enough runs keep every CU busy.  Only the grouping depends on the batch.
    const int32_t upr = (int32_t)std::max<int64_t>(1, (n_units + sb::kTargetRuns - 1) / sb::kTargetRuns);
    // row blocks per wave of the bf16 row tiles: two once the batch has enough 64-row tiles to fill the
    // GPU twice over, else one (fp32: one)
    int64_t tiles64 = 0;
    for (int32_t i = 0; i < n_req; ++i)
        if (n_new[i] * G > sb::kRowsPerWave)
            tiles64 += (int64_t)nkv * ((n_new[i] * G + sb::kRowsPerTile - 1) / sb::kRowsPerTile);
    const int32_t rbn = (dims->dtype == SB_BF16 && tiles64 >= sb::kRowBlocksMinTiles) ? sb::kRowBlocksBf16 : 1;
    int32_t n_part = 0;
    int32_t n_grp = 0;                              // locality groups: a request-head's row tiles, or one run
    int32_t tok0 = 0;                               // the request's first row
    for (int32_t i = 0; i < n_req; tok0 += n_new[i], ++i) {
        const int32_t rows = n_new[i] * G;          // (token, query head of the group) rows
        const int32_t nk = ctx[i] + n_new[i];       // keys visible to the last row
        for (int32_t g = 0; g < nkv; ++g) {
            if (rows <= sb::kRowsPerWave) {
                // one 16-row tile over units of kUnitKeys keys, grouped into runs of upr units; a
                // request that fits one run merges its units itself, else each unit leaves a partial
                const int32_t nu = (nk + sb::kUnitKeys - 1) / sb::kUnitKeys;
                const int32_t p0 = nu > upr ? n_part : -1;
                if (p0 >= 0) {
                    groups.push_back({i, g, 0, rows, p0, nu, tok0, 0});
                    n_part += nu;
                }
                for (int32_t u = 0; u < nu; u += upr) {
                    Item it{};
                    it.v[sb::ITEM_REQ] = i;
                    it.v[sb::ITEM_KVH] = g;
                    it.v[sb::ITEM_MODE] = sb::MODE_RUNS;
                    it.v[sb::ITEM_ROW0] = 0;
                    it.v[sb::ITEM_NROWS] = rows;
                    it.v[sb::ITEM_KB] = u * sb::kUnitKeys;
                    it.v[sb::ITEM_KE] = std::min(nk, (u + upr) * sb::kUnitKeys);
                    it.v[sb::ITEM_PART] = p0 >= 0 ? p0 + u : -1;
                    it.v[sb::ITEM_TOK0] = tok0;
                    it.v[sb::ITEM_CTX] = ctx[i];
                    it.v[sb::ITEM_SLOT0] = (int32_t)slot_base[i];
                    it.cost = it.v[sb::ITEM_KE] - it.v[sb::ITEM_KB];
                    it.lane_cost = it.cost + kItemStartCost;
                    it.grp = n_grp++;
                    items.push_back(it);
                }
            } else {
                // row tiles of 64 x rbn rows; the four waves take rbn 16-row blocks each and share the K/V
                // tiles staged in LDS
                const int32_t rows_grp = n_grp++;
                const int32_t rpt = sb::kRowsPerTile * rbn;
                for (int32_t r0 = 0; r0 < rows; r0 += rpt) {
                    Item it{};
                    const int32_t nr = std::min(rpt, rows - r0);
                    const int32_t last_tok = (r0 + nr - 1) / G;
                    it.v[sb::ITEM_REQ] = i;
                    it.v[sb::ITEM_KVH] = g;
                    it.v[sb::ITEM_MODE] = sb::MODE_ROWS;
                    it.v[sb::ITEM_ROW0] = r0;
                    it.v[sb::ITEM_NROWS] = nr;
                    it.v[sb::ITEM_KB] = 0;
                    it.v[sb::ITEM_KE] = ctx[i] + last_tok + 1;
                    it.v[sb::ITEM_PART] = -1;
                    it.v[sb::ITEM_TOK0] = tok0;
                    it.v[sb::ITEM_CTX] = ctx[i];
                    it.v[sb::ITEM_SLOT0] = (int32_t)slot_base[i];
                    it.v[sb::ITEM_RB] = rbn;
                    it.cost = 4 * (int64_t)it.v[sb::ITEM_KE];
                    it.lane_cost = (int64_t)it.v[sb::ITEM_KE] + kItemStartCost;
                    it.grp = rows_grp;
                    items.push_back(it);
                }
            }
        }
    }
    // Dispatch order.  By default heaviest items first (a row tile weighted 4 x its keys against a run's
    // keys), so the long ones start early and the decode runs and prefill tiles interleave.  When the
    // prefill tiles carry most of the work (long prompts), locality matters more: the row tiles of one
    // request and K/V head re-read the same keys (each up to its own causal limit); workgroups are dealt to
    // the kXcds XCDs round-robin by index, and each XCD has its own L2, so such a group is placed at
    // indices of one residue mod kXcds: its tiles then run side by side on one XCD and share that L2.
    // Groups go to the XCD lanes heaviest first, each to the least loaded lane (estimated cost: keys plus
    // a start-up term); a lane runs its groups in that order, a group's tiles heaviest first.  Lanes are
    // padded to one length with empty items (n_rows 0, skipped by the kernel); if that would take more
    // than a quarter of the items, the heaviest-first order is kept.
    int64_t rows_cost = 0, runs_cost = 0;
    for (const Item& it : items) (it.v[sb::ITEM_MODE] == sb::MODE_ROWS ? rows_cost : runs_cost) += it.lane_cost;
    bool lanes = rows_cost >= runs_cost && rows_cost > 0;
    if (lanes) {
        std::vector<int64_t> gcost(n_grp, 0);
        for (const Item& it : items) gcost[it.grp] += it.lane_cost;
        std::vector<int32_t> gorder(n_grp);
        for (int32_t g = 0; g < n_grp; ++g) gorder[g] = g;
        std::stable_sort(gorder.begin(), gorder.end(), [&](int32_t a, int32_t b) { return gcost[a] > gcost[b]; });
        std::vector<int32_t> lane_of(n_grp), rank_of(n_grp);
        int64_t load[kXcds] = {};
        for (int32_t r = 0; r < n_grp; ++r) {
            const int32_t g = gorder[r];
            int x = 0;
            for (int y = 1; y < kXcds; ++y)
                if (load[y] < load[x]) x = y;
            lane_of[g] = x;
            rank_of[g] = r;
            load[x] += gcost[g];
        }
        std::stable_sort(items.begin(), items.end(), [&](const Item& a, const Item& b) {
            if (a.grp != b.grp) return rank_of[a.grp] < rank_of[b.grp];
            return a.lane_cost > b.lane_cost;
        });
        std::vector<std::vector<int32_t>> lane(kXcds);
        for (int32_t k = 0; k < (int32_t)items.size(); ++k) lane[lane_of[items[k].grp]].push_back(k);
        size_t len = 0;
        for (const auto& l : lane) len = std::max(len, l.size());
        const size_t padded = len * kXcds;
        if (padded - items.size() <= items.size() / 4 + kXcds) {
            std::vector<Item> out(padded);
            for (size_t k = 0; k < len; ++k)
                for (int x = 0; x < kXcds; ++x) {
                    Item& o = out[k * kXcds + x];
                    if (k < lane[x].size()) {
                        o = items[lane[x][k]];
                    } else {
                        o = Item{};
                        o.v[sb::ITEM_MODE] = sb::MODE_ROWS;          // empty: n_rows 0
                        o.v[sb::ITEM_PART] = -1;
                    }
                }
            items.swap(out);
        } else {
            lanes = false;
        }
    }
    if (!lanes)
        std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });

    const Layout L = layout_for(n_req, T, (int64_t)items.size(), (int64_t)groups.size());
    if (L.total * sizeof(int32_t) > bytes)
        return fail(SB_ERR_WORKSPACE, "ragged metadata needs %zu bytes, %zu given", L.total * sizeof(int32_t), bytes);
    int32_t* h = (int32_t*)host_staging;
    int32_t t = 0;
    h[L.cu] = 0;
    for (int32_t i = 0; i < n_req; ++i) {
        h[L.ctx + i] = ctx[i];
        for (int32_t j = 0; j < n_new[i]; ++j, ++t) {
            h[L.pos + t] = ctx[i] + j;
            h[L.slot + t] = (int32_t)(slot_base[i] + ctx[i] + j);
            h[L.ids + t] = token_ids ? token_ids[t] : 0;
        }
        h[L.cu + i + 1] = t;
        h[L.last + i] = t - 1;
    }
    for (size_t k = 0; k < items.size(); ++k)
        std::memcpy(h + L.items + k * sb::kItemInts, items[k].v, sizeof(int32_t) * sb::kItemInts);
    for (size_t k = 0; k < groups.size(); ++k)
        std::memcpy(h + L.groups + k * sb::kGroupInts, groups[k].data(), sizeof(int32_t) * sb::kGroupInts);

    const int32_t* dm = (const int32_t*)dev_meta;
    if (dev_meta && L.total) {
        hipError_t e = hipMemcpyAsync(dev_meta, host_staging, L.total * sizeof(int32_t), hipMemcpyHostToDevice,
                                      (hipStream_t)stream);
        if (e != hipSuccess) return fail(SB_ERR_DEVICE, "ragged metadata copy: %s", hipGetErrorString(e));
    }
    // (with dev_meta == NULL the struct points into host_staging: host-side inspection only)
    const int32_t* base = dev_meta ? dm : h;
    out->n_req = n_req;
    out->n_tokens = (int32_t)T;
    out->n_items = (int32_t)items.size();
    out->n_partials = n_part;
    out->n_groups = (int32_t)groups.size();
    out->max_new = max_new;
    out->cu_seqlens = base + L.cu;
    out->ctx_lens = base + L.ctx;
    out->last_row = base + L.last;
    out->tok_pos = base + L.pos;
    out->tok_slot = base + L.slot;
    out->tok_ids = token_ids ? base + L.ids : nullptr;
    out->items = base + L.items;
    out->groups = base + L.groups;
    return SB_OK;
}
