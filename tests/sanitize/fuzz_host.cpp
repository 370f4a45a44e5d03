// Randomised host-side exercise of the library's allocators and planner,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py (host code only; no GPU, no kernels).
//
// COLD pool ("Paged KV cache" page, Code: append with copy-on-write, fork,
// release): after every operation each page's refcount equals the number of
// live block-table entries that name it, the free stack holds exactly the
// pages with refcount 0 (once each), sequence lengths follow the appends,
// every slot lies at row len % P of the table's page len / P, and a failed
// append changes nothing.
// HOT pool (GraniKV paper, Section 3.2): free ranges and resident slabs tile
// [0, capacity) without overlap, free ranges are merged with their
// neighbours, an unreferenced slab carries its release tick and a referenced
// one none, and a failed allocation changes nothing.
// Planner: random batches (up to 512 groups, ragged lengths, both dtypes)
// through spkv_dispatch, spkv_plan_query and spkv_plan_parts stay inside the
// documented caps and the workspace bound.
//
// Usage: fuzz_host <seed> <rounds>.  Prints "ok" and exits 0, or prints the
// broken invariant and exits 1 (a sanitizer report aborts earlier).
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "spkv.h"

namespace {

std::mt19937_64 rng;

int64_t uni(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }

#define CHECK(cond, ...)                                                      \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "invariant broken at %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                                \
            std::fprintf(stderr, "\n");                                       \
            std::exit(1);                                                     \
        }                                                                     \
    } while (0)

// ---------------------------------------------------------------- COLD ----
struct ColdSnapshot {
    std::vector<int32_t> ref, stack;
    bool operator==(const ColdSnapshot &o) const { return ref == o.ref && stack == o.stack; }
};

ColdSnapshot cold_snapshot(const spkv_cold *c, int32_t pages) {
    spkv_cold_info info{};
    CHECK(spkv_cold_get_info(c, &info) == SPKV_OK, "cold_get_info");
    ColdSnapshot s;
    s.ref.resize((size_t)pages);
    s.stack.resize((size_t)info.num_free);
    if (pages) CHECK(spkv_cold_refcounts(c, s.ref.data()) == SPKV_OK, "cold_refcounts");
    if (info.num_free) CHECK(spkv_cold_free_stack(c, s.stack.data()) == SPKV_OK, "cold_free_stack");
    return s;
}

void cold_check(const spkv_cold *c, int32_t pages, int32_t P, const std::vector<int32_t> &live,
                const std::vector<int64_t> &len) {
    const ColdSnapshot s = cold_snapshot(c, pages);
    std::vector<int32_t> uses((size_t)pages, 0);
    int32_t mb = 1;
    for (int32_t id : live) mb = std::max<int32_t>(mb, (int32_t)((len[(size_t)id] + P - 1) / P));
    if (!live.empty()) {
        std::vector<int32_t> tables(live.size() * (size_t)mb), lens(live.size());
        CHECK(spkv_cold_block_tables(c, live.data(), (int32_t)live.size(), mb, tables.data(), lens.data()) ==
                  SPKV_OK, "block_tables");
        for (size_t i = 0; i < live.size(); ++i) {
            const int64_t L = len[(size_t)live[i]];
            CHECK(lens[i] == L, "seq %d length %d, expected %lld", live[i], lens[i], (long long)L);
            const int32_t nb = (int32_t)((L + P - 1) / P);
            for (int32_t j = 0; j < mb; ++j) {
                const int32_t p = tables[i * (size_t)mb + (size_t)j];
                if (j < nb) {
                    CHECK(p >= 0 && p < pages, "seq %d entry %d = %d", live[i], j, p);
                    uses[(size_t)p] += 1;
                } else {
                    CHECK(p == -1, "seq %d padding %d = %d", live[i], j, p);
                }
            }
        }
    }
    std::set<int32_t> in_stack;
    for (int32_t p : s.stack) {
        CHECK(p >= 0 && p < pages && in_stack.insert(p).second, "free stack entry %d", p);
    }
    for (int32_t p = 0; p < pages; ++p) {
        CHECK(s.ref[(size_t)p] == uses[(size_t)p], "page %d ref %d, table uses %d", p, s.ref[(size_t)p],
              uses[(size_t)p]);
        CHECK((s.ref[(size_t)p] == 0) == (in_stack.count(p) == 1), "page %d ref %d vs free stack", p,
              s.ref[(size_t)p]);
    }
}

void fuzz_cold(int rounds) {
    for (int r = 0; r < rounds; ++r) {
        const int32_t P = (int32_t)std::vector<int>{1, 2, 4, 16}[(size_t)uni(0, 3)];
        const int32_t pages = (int32_t)uni(0, 48);
        std::vector<int32_t> order((size_t)pages);
        for (int32_t i = 0; i < pages; ++i) order[(size_t)i] = i;
        std::shuffle(order.begin(), order.end(), rng);
        spkv_cold *c = nullptr;
        CHECK(spkv_cold_create(pages, P, uni(0, 1) ? order.data() : nullptr, &c) == SPKV_OK, "cold_create");
        std::vector<int32_t> live;
        std::vector<int64_t> len;
        for (int op = 0; op < 200; ++op) {
            const int64_t kind = uni(0, 9);
            if (kind == 0 || live.empty()) {
                int32_t id = -1;
                CHECK(spkv_seq_new(c, &id) == SPKV_OK && id == (int32_t)len.size(), "seq_new %d", id);
                live.push_back(id);
                len.push_back(0);
            } else if (kind <= 6) {
                const int32_t n = (int32_t)uni(1, 8);
                std::vector<int32_t> ids((size_t)n), slots((size_t)n, -7), cows((size_t)(2 * n), -7);
                for (auto &x : ids) x = live[(size_t)uni(0, (int64_t)live.size() - 1)];
                const ColdSnapshot before = cold_snapshot(c, pages);
                int32_t ncow = -1, done = -1;
                const spkv_status st = spkv_cold_append_batch(c, ids.data(), n, slots.data(), cows.data(), &ncow, &done);
                CHECK(st == SPKV_OK || st == SPKV_E_NOMEM, "append status %d", st);
                CHECK(done >= 0 && done <= n && (st != SPKV_OK || done == n), "append done %d of %d", done, n);
                CHECK(ncow >= 0 && ncow <= done, "cow count %d", ncow);
                if (done == 0 && st == SPKV_E_NOMEM)
                    CHECK(cold_snapshot(c, pages) == before, "failed append changed the pool");
                for (int32_t i = 0; i < done; ++i) {
                    const int32_t id = ids[(size_t)i];
                    const int64_t t = len[(size_t)id];
                    CHECK(slots[(size_t)i] % P == (int32_t)(t % P), "slot row %d at len %lld", slots[(size_t)i],
                          (long long)t);
                    len[(size_t)id] = t + 1;
                }
                for (int32_t k = 0; k < ncow; ++k) {
                    const int32_t src = cows[(size_t)(2 * k)], dst = cows[(size_t)(2 * k + 1)];
                    CHECK(src >= 0 && src < pages && dst >= 0 && dst < pages && src != dst, "cow pair %d %d", src, dst);
                }
                // every completed slot sits in its sequence's current table at row len % P
                for (int32_t i = 0; i < done; ++i) {
                    const int32_t id = ids[(size_t)i];
                    const int32_t mb = (int32_t)((len[(size_t)id] + P - 1) / P);
                    std::vector<int32_t> tab((size_t)mb);
                    int32_t l = -1;
                    CHECK(spkv_cold_block_tables(c, &id, 1, mb, tab.data(), &l) == SPKV_OK, "table of %d", id);
                    bool found = false;
                    for (int32_t p : tab) found = found || p == slots[(size_t)i] / P;
                    CHECK(found, "slot %d of seq %d is not in its table", slots[(size_t)i], id);
                }
            } else if (kind <= 8) {
                const int32_t src = live[(size_t)uni(0, (int64_t)live.size() - 1)];
                int32_t dst = -1;
                CHECK(spkv_cold_fork(c, src, &dst) == SPKV_OK && dst == (int32_t)len.size(), "fork");
                live.push_back(dst);
                len.push_back(len[(size_t)src]);
            } else {
                const size_t i = (size_t)uni(0, (int64_t)live.size() - 1);
                CHECK(spkv_cold_release(c, live[i]) == SPKV_OK, "release");
                CHECK(spkv_cold_release(c, live[i]) == SPKV_E_STATE, "second release");
                live.erase(live.begin() + (std::ptrdiff_t)i);
            }
            cold_check(c, pages, P, live, len);
        }
        for (int32_t id : live) CHECK(spkv_cold_release(c, id) == SPKV_OK, "teardown release");
        spkv_cold_info info{};
        CHECK(spkv_cold_get_info(c, &info) == SPKV_OK && info.num_free == pages && info.num_live == 0,
              "teardown: %d of %d pages free", info.num_free, pages);
        spkv_cold_destroy(c);
    }
}

// ----------------------------------------------------------------- HOT ----
struct HotSnapshot {
    std::vector<int64_t> fb, fl, sb, sl, lru;
    std::vector<int32_t> ref;
    bool operator==(const HotSnapshot &o) const {
        return fb == o.fb && fl == o.fl && sb == o.sb && sl == o.sl && lru == o.lru && ref == o.ref;
    }
};

HotSnapshot hot_snapshot(const spkv_hot *h) {
    spkv_hot_info info{};
    CHECK(spkv_hot_get_info(h, &info) == SPKV_OK, "hot_get_info");
    HotSnapshot s;
    const int32_t nf = info.num_free_ranges, ns = info.num_slabs;
    s.fb.resize((size_t)nf);
    s.fl.resize((size_t)nf);
    s.sb.resize((size_t)ns);
    s.sl.resize((size_t)ns);
    s.lru.resize((size_t)ns);
    s.ref.resize((size_t)ns);
    CHECK(spkv_hot_free_ranges(h, s.fb.data(), s.fl.data(), nf) == SPKV_OK, "free_ranges");
    CHECK(spkv_hot_slabs(h, s.sb.data(), s.sl.data(), s.ref.data(), s.lru.data(), ns) == SPKV_OK, "slabs");
    return s;
}

void hot_check(const spkv_hot *h, int64_t cap) {
    const HotSnapshot s = hot_snapshot(h);
    std::vector<std::pair<int64_t, int64_t>> all;   // (base, len), tagged by sign of len for free
    for (size_t i = 0; i < s.fb.size(); ++i) {
        CHECK(s.fl[i] > 0, "empty free range");
        if (i) CHECK(s.fb[i - 1] + s.fl[i - 1] < s.fb[i], "free ranges %zu, %zu overlap or touch", i - 1, i);
        all.push_back({s.fb[i], s.fl[i]});
    }
    for (size_t i = 0; i < s.sb.size(); ++i) {
        CHECK(s.sl[i] > 0 && s.ref[i] >= 0, "slab %zu len %lld ref %d", i, (long long)s.sl[i], s.ref[i]);
        CHECK((s.ref[i] > 0) == (s.lru[i] == -1), "slab %zu ref %d lru %lld", i, s.ref[i], (long long)s.lru[i]);
        all.push_back({s.sb[i], s.sl[i]});
    }
    std::sort(all.begin(), all.end());
    int64_t at = 0;
    for (auto &r : all) {
        CHECK(r.first == at, "gap or overlap at %lld (next range at %lld)", (long long)at, (long long)r.first);
        at += r.second;
    }
    CHECK(at == cap, "ranges cover %lld of %lld", (long long)at, (long long)cap);
}

void fuzz_hot(int rounds) {
    for (int r = 0; r < rounds; ++r) {
        const int64_t cap = uni(0, 400);
        spkv_hot *h = nullptr;
        CHECK(spkv_hot_create(cap, &h) == SPKV_OK, "hot_create");
        for (int op = 0; op < 200; ++op) {
            const HotSnapshot s = hot_snapshot(h);
            const int64_t kind = uni(0, 9);
            if (kind <= 3) {
                const int64_t lp = uni(1, std::max<int64_t>(1, cap / 3));
                int64_t base = -1;
                const spkv_status st = spkv_hot_alloc(h, lp, &base);
                CHECK(st == SPKV_OK || st == SPKV_E_NOMEM, "hot_alloc status %d", st);
                if (st == SPKV_E_NOMEM) CHECK(hot_snapshot(h) == s, "failed alloc changed the pool");
                else CHECK(base >= 0 && base + lp <= cap, "slab [%lld, +%lld)", (long long)base, (long long)lp);
            } else if (kind <= 5 && !s.sb.empty()) {
                const size_t i = (size_t)uni(0, (int64_t)s.sb.size() - 1);
                CHECK(spkv_hot_incref(h, s.sb[i]) == SPKV_OK, "incref");
            } else if (kind <= 8 && !s.sb.empty()) {
                const size_t i = (size_t)uni(0, (int64_t)s.sb.size() - 1);
                const spkv_status st = spkv_hot_decref(h, s.sb[i]);
                CHECK(st == (s.ref[i] > 0 ? SPKV_OK : SPKV_E_STATE), "decref of ref %d gave %d", s.ref[i], st);
            } else if (kind == 9) {
                int32_t n = -1;
                CHECK(spkv_hot_evict_unreferenced(h, &n) == SPKV_OK && n >= 0, "evict");
            }
            CHECK(spkv_hot_decref(h, cap + 5) == SPKV_E_STATE, "decref of no slab");
            hot_check(h, cap);
        }
        spkv_hot_destroy(h);
    }
}

// ------------------------------------------------------------- planner ----
void fuzz_plan(int rounds) {
    for (int r = 0; r < rounds; ++r) {
        const int32_t hkv = (int32_t)uni(1, 16), G = (int32_t)uni(1, 8);
        const int32_t B = (int32_t)(uni(0, 3) == 0 ? uni(0, 3) : uni(1, 600));
        const int32_t ng = (int32_t)uni(0, 512);
        const int32_t P = uni(0, 1) ? 1 : 16;
        std::vector<int32_t> group_of((size_t)B), hot_len((size_t)ng), cold_lens((size_t)B);
        std::vector<int64_t> hot_base((size_t)ng);
        int64_t at = 0;
        for (int32_t g = 0; g < ng; ++g) {
            hot_len[(size_t)g] = (int32_t)(uni(0, 4) == 0 ? uni(0, 40) : uni(1, 40000));
            hot_base[(size_t)g] = at;
            at += hot_len[(size_t)g];
        }
        int32_t max_len = 0;
        for (int32_t b = 0; b < B; ++b) {
            group_of[(size_t)b] = ng == 0 ? -1 : (int32_t)uni(-1, ng - 1);
            cold_lens[(size_t)b] = (int32_t)(uni(0, 9) == 0 ? 0 : uni(1, 5000));
            max_len = std::max(max_len, cold_lens[(size_t)b]);
        }
        const int32_t mb = (max_len + P - 1) / P + 1;
        std::vector<int32_t> tables((size_t)B * (size_t)mb, -1);
        std::vector<uint16_t> q((size_t)B * (size_t)(hkv * G) * 128 + 1);
        spkv_batch b{};
        b.batch = B;
        b.num_q_heads = hkv * G;
        b.num_kv_heads = hkv;
        b.head_dim = uni(0, 1) ? 64 : 128;
        b.dtype = uni(0, 3) ? SPKV_DTYPE_BF16 : SPKV_DTYPE_F32;
        b.scale = 0.125f;
        b.q = q.data();                       // host arrays stand in for device pointers:
        b.num_groups = ng;                    // the planner must not read them
        b.group_of = group_of.data();
        b.hot_base = hot_base.data();
        b.hot_len = hot_len.data();
        b.host_group_of = group_of.data();
        b.host_hot_base = hot_base.data();
        b.host_hot_len = hot_len.data();
        b.page_size = P;
        b.max_blocks = mb;
        b.block_tables = tables.data();
        b.cold_lens = cold_lens.data();
        b.host_cold_lens = cold_lens.data();

        const size_t ws = spkv_workspace_size(&b);
        CHECK(ws > 0, "workspace_size 0 for a valid batch");
        std::vector<int32_t> choice((size_t)std::max(1, ng), -1);
        spkv_dispatch_params prm{};
        spkv_dispatch_params_default(&prm);
        for (int32_t mode = 0; mode < 4; ++mode) {
            prm.mode = mode;
            CHECK(spkv_dispatch(&b, &prm, choice.data()) == SPKV_OK, "dispatch mode %d", mode);
            for (int32_t g = 0; g < ng; ++g) CHECK(choice[(size_t)g] == 0 || choice[(size_t)g] == 1, "choice");
            if (mode == SPKV_MODE_FORCE_DENSE)
                for (int32_t g = 0; g < ng; ++g) CHECK(choice[(size_t)g] == 0, "forced dense chose cascade");
            spkv_plan_info info{};
            CHECK(spkv_plan_query(&b, choice.data(), &info) == SPKV_OK, "plan_query");
            CHECK(info.workspace_bytes >= 0 && (size_t)info.workspace_bytes <= ws, "plan needs %lld > bound %zu",
                  (long long)info.workspace_bytes, ws);
            CHECK(info.flat_splits <= info.flat_split_cap && info.prefix_splits <= info.prefix_split_cap,
                  "splits beyond caps");
            std::vector<int32_t> fp((size_t)std::max(1, B), -1), pp((size_t)std::max(1, B), -1);
            CHECK(spkv_plan_parts(&b, choice.data(), fp.data(), pp.data()) == SPKV_OK, "plan_parts");
            for (int32_t i = 0; i < B; ++i) {
                const int32_t g = group_of[(size_t)i];
                const bool casc = g >= 0 && choice[(size_t)g] == 1 && hot_len[(size_t)g] > 0;
                const int64_t paged = cold_lens[(size_t)i] + (g >= 0 && !casc ? hot_len[(size_t)g] : 0);
                CHECK(fp[(size_t)i] >= 0 && fp[(size_t)i] <= info.flat_splits, "flat parts %d of %d", fp[(size_t)i],
                      info.flat_splits);
                CHECK((fp[(size_t)i] > 0) == (paged > 0), "request %d: %d paged parts for %lld tokens", i,
                      fp[(size_t)i], (long long)paged);
                CHECK(pp[(size_t)i] >= 0 && pp[(size_t)i] <= info.prefix_splits, "prefix parts %d", pp[(size_t)i]);
                CHECK((pp[(size_t)i] > 0) == casc, "request %d: %d prefix parts, cascade %d", i, pp[(size_t)i],
                      (int)casc);
            }
        }
        // an invalid group index is refused
        if (B > 0) {
            group_of[0] = ng;
            CHECK(spkv_dispatch(&b, &prm, choice.data()) == SPKV_E_INVAL, "group index %d accepted", ng);
            CHECK(spkv_workspace_size(&b) == 0, "workspace for an invalid batch");
        }
    }
}

}  // namespace

int main(int argc, char **argv) {
    const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int rounds = argc > 2 ? std::atoi(argv[2]) : 20;
    rng.seed(seed);
    fuzz_cold(rounds);
    fuzz_hot(rounds);
    fuzz_plan(rounds);
    std::printf("ok\n");
    return 0;
}
