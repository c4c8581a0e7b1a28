// Host-only driver of libsb's C ABI for a sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer): exercises the K/V manager, the iteration-level
// scheduler in each of its modes, and the ragged metadata builder, all without a
// GPU (bookkeeping-only K/V manager, dev_meta = NULL), and checks the invariants
// that the scheduling rules fix along the way:
//   - reservations are disjoint, 8-aligned, inside the arena, and their total is
//     the manager's counter, never above n_slots (the slot constraint of the
//     iteration-level FCFS pages: a request reserves max_tokens when first
//     scheduled, and admission fails iff the counter would pass n_slots);
//   - a batch never exceeds max_bs; every request ends with out_len tokens, which
//     are the values the driver fed back;
//   - the ragged metadata's offsets, positions and slots follow Split / Merge as
//     offsets (request i owns rows cu[i]..cu[i+1]-1; its j-th new token sits at
//     position ctx_i + j and slot slot_base_i + ctx_i + j).
// Exit status 0 and no sanitizer report means the run was clean.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <map>
#include <random>
#include <vector>

#include "sb.h"

static int g_fail = 0;
#define CHECK(c)                                                                        \
    do {                                                                                \
        if (!(c)) {                                                                     \
            std::fprintf(stderr, "CHECK failed %s:%d: %s (%s)\n", __FILE__, __LINE__, #c, \
                         sb_last_error());                                              \
            ++g_fail;                                                                   \
            return;                                                                     \
        }                                                                               \
    } while (0)
#define OK(e) CHECK((e) == SB_OK)

// ------------------------------------------------------------------ K/V manager
static void kv_random(uint32_t seed) {
    std::mt19937 rng(seed);
    const int64_t n_slots = 4096;
    const int32_t max_live = 48;
    const int64_t arena = sb_kv_arena_slots(n_slots, max_live);
    CHECK(arena >= n_slots);
    sb_kv* kv = nullptr;
    OK(sb_kv_create(n_slots, arena, 2, 2, 64, SB_BF16, nullptr, nullptr, &kv));
    std::map<int64_t, std::pair<int64_t, int32_t>> live;   // id -> (base, max_tokens)
    int64_t next_id = 0;
    for (int step = 0; step < 4000; ++step) {
        const bool add = live.empty() || ((int)live.size() < max_live && rng() % 100 < 55);
        if (add) {
            const int32_t mt = 1 + (int32_t)(rng() % (rng() % 4 == 0 ? 1024 : 96));
            int64_t base = -1;
            int64_t rsrv = 0;
            for (auto& kvp : live) rsrv += kvp.second.second;
            const int st = sb_kv_reserve(kv, next_id, mt, &base);
            if (rsrv + mt > n_slots) {
                CHECK(st == SB_ERR_NO_SLOTS);
            } else {
                OK(st);
                CHECK(base >= 0 && base % 8 == 0 && base + mt <= arena);
                live[next_id] = {base, mt};
            }
            ++next_id;
        } else {
            auto it = live.begin();
            std::advance(it, rng() % live.size());
            OK(sb_kv_free(kv, it->first));
            CHECK(sb_kv_free(kv, it->first) == SB_ERR_NOT_FOUND);
            live.erase(it);
        }
        // compaction may move every live range: re-read them all
        std::vector<std::pair<int64_t, int64_t>> ranges;
        int64_t rsrv = 0;
        for (auto& kvp : live) {
            int64_t b;
            int32_t m;
            OK(sb_kv_lookup(kv, kvp.first, &b, &m));
            CHECK(m == kvp.second.second && b % 8 == 0 && b >= 0 && b + m <= arena);
            kvp.second.first = b;
            ranges.push_back({b, b + m});
            rsrv += m;
        }
        std::sort(ranges.begin(), ranges.end());
        for (size_t i = 1; i < ranges.size(); ++i) CHECK(ranges[i - 1].second <= ranges[i].first);
        int64_t c_rsrv, c_slots, c_live, c_comp;
        OK(sb_kv_stats(kv, &c_rsrv, &c_slots, &c_live, &c_comp));
        CHECK(c_rsrv == rsrv && c_slots == n_slots && c_live == (int64_t)live.size() && c_rsrv <= n_slots);
    }
    // error paths
    int64_t b;
    int32_t m;
    CHECK(sb_kv_reserve(kv, -5, (int32_t)n_slots + 1, &b) == SB_ERR_TOO_LARGE ||
          sb_kv_reserve(kv, -5, (int32_t)n_slots + 1, &b) == SB_ERR_NO_SLOTS);
    CHECK(sb_kv_lookup(kv, -12345, &b, &m) == SB_ERR_NOT_FOUND);
    CHECK(sb_kv_reserve(kv, 0, 0, &b) != SB_OK);
    CHECK(sb_kv_reserve(nullptr, 0, 1, &b) == SB_ERR_INVALID);
    sb_kv_destroy(kv);
    sb_kv_destroy(nullptr);
}

// ------------------------------------------------------------------ ragged metadata
static void check_ragged(const sb_model_dims& d, int32_t n, const int32_t* n_new, const int32_t* ctx,
                         const int64_t* base, const int32_t* toks) {
    int64_t T = 0, keys = 0;
    for (int32_t i = 0; i < n; ++i) T += n_new[i], keys += ctx[i] + n_new[i];
    const size_t bytes = sb_ragged_bytes(&d, n, (int32_t)T, keys);
    CHECK(bytes > 0 || n == 0);
    // exact-size heap buffer: an overrun is an ASan report
    std::vector<int32_t> staging((bytes + 3) / 4 + (bytes == 0));
    sb_ragged rg;
    std::memset(&rg, 0, sizeof rg);
    OK(sb_ragged_build(&d, n, n_new, ctx, base, toks, staging.data(), nullptr, bytes, nullptr, &rg));
    CHECK(rg.n_req == n && rg.n_tokens == (int32_t)T);
    CHECK(rg.n_partials <= sb_attn_max_partials(&d, n, keys));
    CHECK(rg.cu_seqlens[0] == 0);
    for (int32_t i = 0; i < n; ++i) {
        CHECK(rg.cu_seqlens[i + 1] - rg.cu_seqlens[i] == n_new[i]);
        CHECK(rg.ctx_lens[i] == ctx[i] && rg.last_row[i] == rg.cu_seqlens[i + 1] - 1);
        for (int32_t j = 0; j < n_new[i]; ++j) {
            const int32_t r = rg.cu_seqlens[i] + j;
            CHECK(rg.tok_pos[r] == ctx[i] + j);
            CHECK(rg.tok_slot[r] == base[i] + ctx[i] + j);
            if (toks) CHECK(rg.tok_ids[r] == toks[r]);
        }
    }
    // sb_ragged_bytes is an upper bound: find the exact need (the smallest size the
    // builder accepts), then build into a heap buffer of exactly that size, so a
    // write beyond what the size check allowed is a sanitizer report; one int less
    // must be refused with SB_ERR_WORKSPACE, not overrun
    size_t lo = 0, hi = bytes;   // build(hi) succeeds
    while (hi - lo > 4) {
        const size_t mid = (lo + hi) / 2 / 4 * 4;
        std::vector<int32_t> probe(mid / 4 + 1);
        const int st = sb_ragged_build(&d, n, n_new, ctx, base, toks, probe.data(), nullptr, mid, nullptr, &rg);
        CHECK(st == SB_OK || st == SB_ERR_WORKSPACE);
        (st == SB_OK ? hi : lo) = mid;
    }
    if (hi > 0) {
        int32_t* exact = new int32_t[hi / 4];
        OK(sb_ragged_build(&d, n, n_new, ctx, base, toks, exact, nullptr, hi, nullptr, &rg));
        CHECK(rg.n_tokens == (int32_t)T && (n == 0 || rg.cu_seqlens[n] == (int32_t)T));
        const int st = sb_ragged_build(&d, n, n_new, ctx, base, toks, exact, nullptr, hi - 4, nullptr, &rg);
        delete[] exact;
        CHECK(st == SB_ERR_WORKSPACE);
    }
}

// ------------------------------------------------------------------ scheduler
enum Mode { SYNC, DEFERRED, CHUNKED, REQUEST_LEVEL };

static void sched_random(uint32_t seed, Mode mode, const sb_model_dims& d) {
    std::mt19937 rng(seed);
    const int64_t n_slots = 3000;
    const int32_t max_bs = 1 + (int32_t)(rng() % 16);
    sb_kv* kv = nullptr;
    OK(sb_kv_create(n_slots, sb_kv_arena_slots(n_slots, 64), d.n_layers, d.n_kv_heads, d.head_dim, d.dtype,
                    nullptr, nullptr, &kv));
    sb_sched* s = nullptr;
    OK(sb_sched_create(max_bs, kv, &s));
    if (mode == CHUNKED) OK(sb_sched_set_chunking(s, 64 + (int32_t)(rng() % 200), 8 + (int32_t)(rng() % 64)));
    if (mode == REQUEST_LEVEL) OK(sb_sched_set_request_level(s, 1));

    struct Req { int32_t plen, out_len; std::vector<int32_t> fed; };
    std::map<int64_t, Req> reqs;
    const int n_req = 120;
    for (int64_t id = 0; id < n_req; ++id) {
        Req r;
        r.plen = 1 + (int32_t)(rng() % (rng() % 5 == 0 ? 400 : 40));
        r.out_len = 1 + (int32_t)(rng() % 30);
        int32_t mt = 0;
        OK(sb_reservation_tokens((int32_t)(id % 3), r.plen, r.out_len, 64, &mt));
        std::vector<int32_t> prompt(r.plen);
        for (auto& t : prompt) t = (int32_t)(rng() % d.vocab);
        if (mode == SYNC && id % 10 == 9 && r.out_len >= 2) {
            // a request that already generated `gen` tokens elsewhere: its output starts as
            // gen - 1 zeros (values the scheduler never saw) followed by last_token
            const int32_t gen = 1 + (int32_t)(rng() % (r.out_len - 1));
            const int32_t last = (int32_t)(rng() % d.vocab);
            const int st = sb_sched_add_running(s, id, (double)id, r.plen, prompt.data(), r.out_len, mt, gen, last);
            if (st == SB_ERR_NO_SLOTS) continue;
            OK(st);
            r.fed.assign(gen, 0);
            r.fed.back() = last;
        } else {
            OK(sb_sched_add(s, id, (double)id, r.plen, prompt.data(), r.out_len, mt));
        }
        reqs[id] = r;
    }
    std::vector<int64_t> ids(max_bs), fin(max_bs);
    std::vector<int32_t> nn(max_bs), cx(max_bs), tok(max_bs);
    std::vector<int64_t> base(max_bs);
    std::vector<int32_t> toks(1 << 16);
    int64_t ticket_pending = -1;
    std::vector<int32_t> pending_vals;
    int finished = 0, iters = 0;
    while (iters < 100000) {
        int32_t n = 0;
        OK(sb_select_batch(s, max_bs, ids.data(), nn.data(), cx.data(), base.data(), &n));
        CHECK(n <= max_bs);
        if (n == 0) break;
        ++iters;
        // every base handed out is the manager's current one (a reservation made during this Select may
        // have compacted the arena and moved the members admitted before it)
        for (int32_t i = 0; i < n; ++i) {
            int64_t lb = -1;
            OK(sb_kv_lookup(kv, ids[i], &lb, nullptr));
            CHECK(lb == base[i]);
        }
        int64_t reserved = 0, stored = 0;
        OK(sb_kv_usage(s, &reserved, &stored));
        CHECK(reserved <= n_slots && stored <= reserved);
        int32_t nt = 0;
        int64_t ref_ticket = -1;
        if (mode == DEFERRED) {
            // settle the previous iteration's values only after this batch's refs were taken
            OK(sb_batch_token_refs(s, n, ids.data(), (int32_t)toks.size(), toks.data(), &nt, &ref_ticket));
            CHECK(ref_ticket == -1 || ref_ticket == ticket_pending);
            if (ticket_pending >= 0) {
                OK(sb_sched_set_tokens(s, ticket_pending, (int32_t)pending_vals.size(), pending_vals.data()));
                CHECK(sb_sched_set_tokens(s, ticket_pending, (int32_t)pending_vals.size(), pending_vals.data()) ==
                      SB_ERR_NOT_FOUND);
                ticket_pending = -1;
            }
            int32_t nt2 = 0;
            OK(sb_batch_tokens(s, n, ids.data(), (int32_t)toks.size(), toks.data(), &nt2));
            CHECK(nt2 == nt);
        } else {
            OK(sb_batch_tokens(s, n, ids.data(), (int32_t)toks.size(), toks.data(), &nt));
        }
        int32_t sum = 0;
        for (int32_t i = 0; i < n; ++i) sum += nn[i];
        CHECK(sum == nt);
        // the ragged metadata of this very batch
        check_ragged(d, n, nn.data(), cx.data(), base.data(), toks.data());
        if (g_fail) return;
        for (int32_t i = 0; i < n; ++i) tok[i] = (int32_t)((ids[i] * 131 + iters) % d.vocab);
        int32_t nf = 0;
        if (mode == DEFERRED) {
            int64_t ticket = -1;
            OK(sb_sched_complete_deferred(s, n, ids.data(), &nf, fin.data(), &ticket));
            ticket_pending = ticket;
            pending_vals.assign(tok.begin(), tok.begin() + n);
        } else {
            OK(sb_sched_complete(s, n, ids.data(), tok.data(), &nf, fin.data()));
        }
        // a member yields a token unless it fed a non-final prompt chunk (chunked prefill)
        for (int32_t i = 0; i < n; ++i) {
            Req& r = reqs[ids[i]];
            const bool yields = mode != CHUNKED || cx[i] + nn[i] >= r.plen;
            if (yields) r.fed.push_back(tok[i]);
        }
        finished += nf;
    }
    if (ticket_pending >= 0)
        OK(sb_sched_set_tokens(s, ticket_pending, (int32_t)pending_vals.size(), pending_vals.data()));
    CHECK(finished == (int)reqs.size());
    int32_t pool = -1;
    int64_t rsrv = -1, nfin = -1;
    OK(sb_sched_stats(s, &pool, &rsrv, &nfin));
    CHECK(pool == 0 && rsrv == 0 && nfin == (int64_t)reqs.size());
    std::vector<int32_t> out(64);
    for (auto& kvp : reqs) {
        int32_t n = 0;
        OK(sb_sched_output(s, kvp.first, (int32_t)out.size(), out.data(), &n));
        CHECK(n == kvp.second.out_len && (size_t)n == kvp.second.fed.size());
        for (int32_t j = 0; j < n; ++j) CHECK(out[j] == kvp.second.fed[j]);
        if (n > 1) CHECK(sb_sched_output(s, kvp.first, n - 1, out.data(), &n) == SB_ERR_CAPACITY);
    }
    sb_sched_destroy(s);
    sb_kv_destroy(kv);
}

static void ragged_edges(const sb_model_dims& d) {
    // empty batch
    check_ragged(d, 0, nullptr, nullptr, nullptr, nullptr);
    // one long prefill next to many decodes, ragged tails everywhere
    std::vector<int32_t> nn, cx;
    std::vector<int64_t> base;
    int64_t b = 0;
    nn.push_back(1000), cx.push_back(0), base.push_back(b), b += 1008;
    for (int i = 0; i < 37; ++i) {
        nn.push_back(1), cx.push_back(1 + 97 * i), base.push_back(b);
        b += ((2 + 97 * i) + 7) / 8 * 8;
    }
    nn.push_back(65), cx.push_back(300), base.push_back(b);
    check_ragged(d, (int32_t)nn.size(), nn.data(), cx.data(), base.data(), nullptr);
    // rejected inputs leave no overrun behind
    std::vector<int32_t> st(64);
    sb_ragged rg;
    int32_t bad_new = 0, c0 = 0;
    int64_t b0 = 0, b_odd = 3;
    int32_t one = 1;
    CHECK(sb_ragged_build(&d, 1, &bad_new, &c0, &b0, nullptr, st.data(), nullptr, 256, nullptr, &rg) ==
          SB_ERR_INVALID);
    CHECK(sb_ragged_build(&d, 1, &one, &c0, &b_odd, nullptr, st.data(), nullptr, 256, nullptr, &rg) ==
          SB_ERR_INVALID);
    int32_t tok_bad = d.vocab;
    CHECK(sb_ragged_build(&d, 1, &one, &c0, &b0, &tok_bad, st.data(), nullptr, 256, nullptr, &rg) ==
          SB_ERR_INVALID);
    CHECK(sb_ragged_build(&d, 1, &one, &c0, &b0, nullptr, nullptr, nullptr, 256, nullptr, &rg) == SB_ERR_INVALID);
}

int main() {
    sb_model_dims llama = {SB_ARCH_LLAMA, SB_BF16, 2, 256, 8, 2, 32, 512, 1000, 0, 1e-5f, 10000.0f};
    sb_model_dims gpt = {SB_ARCH_GPT, SB_BF16, 2, 256, 4, 4, 64, 1024, 1000, 4096, 1e-5f, 0.0f};
    for (uint32_t seed = 0; seed < 3; ++seed) kv_random(seed);
    for (const sb_model_dims* d : {&llama, &gpt}) {
        ragged_edges(*d);
        for (uint32_t seed = 0; seed < 2; ++seed)
            for (Mode m : {SYNC, DEFERRED, CHUNKED, REQUEST_LEVEL}) sched_random(100 + seed, m, *d);
    }
    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("host driver: all checks passed\n");
    return 0;
}
