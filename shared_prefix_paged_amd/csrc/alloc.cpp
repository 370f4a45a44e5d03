// Host allocators behind the C ABI: COLD page pool and HOT slab pool.
//
// COLD: "Paged KV cache" page, How it works and Code - fixed-size pages with
// per-page refcounts, a LIFO free stack, per-sequence tables, append with
// copy-on-write, fork and release.  The page fixes 16 tokens per page; here it
// is a parameter (the GraniKV paper's COLD pool uses 1, its Section 3.3).
//
// HOT: GraniKV paper, Section 3.2 - one contiguous range of Lp token slots per
// prefix, first fit over address-ordered free ranges, unreferenced slabs
// evicted least-recently-released first with the freed range merged into its
// free neighbours; Appendix B.10 - a prefix that does not fit is reported so
// the caller can keep it in the COLD pool.
#include <algorithm>
#include <map>
#include <utility>
#include <vector>

#include "internal.h"

struct spkv_cold {
    struct Seq {
        std::vector<int32_t> table;
        int32_t len = 0;
        bool live = true;
    };
    int32_t num_pages = 0;
    int32_t page_size = 1;
    std::vector<int32_t> ref;
    std::vector<int32_t> stack;   // bottom -> top; back() is handed out next
    std::vector<Seq> seqs;        // index = id
    int32_t live = 0;
};

struct spkv_hot {
    struct Slab {
        int64_t len;
        int32_t ref;
        int64_t lru;              // -1 while referenced
    };
    int64_t capacity = 0;
    std::vector<std::pair<int64_t, int64_t>> free;   // (base, len), ascending, merged
    std::map<int64_t, Slab> slabs;                     // by base
    int64_t tick = 0;
};

namespace {

using spkv::fail;

// ---- COLD -----------------------------------------------------------------

spkv_cold::Seq *live_seq(spkv_cold *c, int32_t id) {
    if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].live) return nullptr;
    return &c->seqs[id];
}

// Where the next token of a sequence goes.  Token t belongs to page t / P of
// the sequence at row t % P.  A sequence writes only into pages it owns
// alone: when that page does not exist yet (t starts a page) or is still
// referenced by another sequence (after a fork), a page must come off the
// free stack first; in the second case the shared page is swapped for the new
// one, whose first rows the caller fills with a copy of the old page.
struct NextSlot {
    int32_t page_index = 0;   // position in the sequence's table
    int32_t row = 0;          // row inside the page
    bool needs_page = false;  // a page comes off the free stack
    int32_t replaced = -1;    // shared page being swapped out, or -1
};

NextSlot next_slot(const spkv_cold *c, const spkv_cold::Seq &s) {
    NextSlot n;
    n.page_index = s.len / c->page_size;
    n.row = s.len % c->page_size;
    if (n.page_index == (int32_t)s.table.size()) {
        n.needs_page = true;
    } else {
        const int32_t cur = s.table[(size_t)n.page_index];
        if (c->ref[(size_t)cur] > 1) {
            n.needs_page = true;
            n.replaced = cur;
        }
    }
    return n;
}

int32_t take_page(spkv_cold *c) {
    const int32_t pg = c->stack.back();
    c->stack.pop_back();
    c->ref[(size_t)pg] = 1;
    return pg;
}

// Reserve a slot for the token at position len of sequence id.  The decision
// is made first and checked against the free stack, then applied in one go,
// so a failure (no free page) leaves every piece of state untouched.
spkv_status cold_append_one(spkv_cold *c, int32_t id, int32_t *slot, int32_t *cow_src, int32_t *cow_dst) {
    spkv_cold::Seq *s = live_seq(c, id);
    if (!s) return fail(SPKV_E_STATE, "append: unknown or released sequence " + std::to_string(id));
    const NextSlot n = next_slot(c, *s);
    if (n.needs_page && c->stack.empty())
        return fail(SPKV_E_NOMEM, n.replaced >= 0 ? "COLD pool exhausted (copy-on-write)" : "COLD pool exhausted");
    *cow_src = -1;
    *cow_dst = -1;
    if (n.needs_page) {
        const int32_t fresh = take_page(c);
        if (n.replaced >= 0) {
            s->table[(size_t)n.page_index] = fresh;
            c->ref[(size_t)n.replaced] -= 1;   // still >= 1: another sequence holds it
            *cow_src = n.replaced;
            *cow_dst = fresh;
        } else {
            s->table.push_back(fresh);
        }
    }
    *slot = s->table[(size_t)n.page_index] * c->page_size + n.row;
    s->len += 1;
    return SPKV_OK;
}

// ---- HOT ------------------------------------------------------------------

void insert_range(std::vector<std::pair<int64_t, int64_t>> &fr, int64_t base, int64_t len) {
    auto it = std::lower_bound(fr.begin(), fr.end(), std::make_pair(base, (int64_t)0));
    it = fr.insert(it, {base, len});
    size_t i = (size_t)(it - fr.begin());
    if (i + 1 < fr.size() && fr[i].first + fr[i].second == fr[i + 1].first) {
        fr[i].second += fr[i + 1].second;
        fr.erase(fr.begin() + (long)i + 1);
    }
    if (i > 0 && fr[i - 1].first + fr[i - 1].second == fr[i].first) {
        fr[i - 1].second += fr[i].second;
        fr.erase(fr.begin() + (long)i);
    }
}

bool first_fit(std::vector<std::pair<int64_t, int64_t>> &fr, int64_t lp, int64_t *base) {
    for (size_t i = 0; i < fr.size(); ++i) {
        if (fr[i].second >= lp) {
            *base = fr[i].first;
            if (fr[i].second == lp) {
                fr.erase(fr.begin() + (long)i);
            } else {
                fr[i].first += lp;
                fr[i].second -= lp;
            }
            return true;
        }
    }
    return false;
}

std::vector<int64_t> lru_order(const spkv_hot *h) {
    std::vector<std::pair<int64_t, int64_t>> c;   // (lru tick, base)
    for (const auto &kv : h->slabs)
        if (kv.second.ref == 0) c.push_back({kv.second.lru, kv.first});
    std::sort(c.begin(), c.end());
    std::vector<int64_t> out;
    for (auto &p : c) out.push_back(p.second);
    return out;
}

}  // namespace

extern "C" {

// ============================== COLD ========================================

spkv_status spkv_cold_create(int32_t num_pages, int32_t page_size, const int32_t *free_order, spkv_cold **out) {
    if (!out) return fail(SPKV_E_INVAL, "cold_create: null out");
    if (num_pages < 0 || page_size < 1) return fail(SPKV_E_INVAL, "cold_create: bad num_pages/page_size");
    if ((int64_t)num_pages * page_size > INT32_MAX) return fail(SPKV_E_INVAL, "cold_create: slot count overflows int32");
    auto *c = new spkv_cold();
    c->num_pages = num_pages;
    c->page_size = page_size;
    c->ref.assign((size_t)num_pages, 0);
    c->stack.resize((size_t)num_pages);
    if (free_order) {
        std::vector<char> seen((size_t)num_pages, 0);
        for (int32_t i = 0; i < num_pages; ++i) {
            int32_t p = free_order[i];
            if (p < 0 || p >= num_pages || seen[(size_t)p]) {
                delete c;
                return fail(SPKV_E_INVAL, "cold_create: free_order is not a permutation");
            }
            seen[(size_t)p] = 1;
            c->stack[(size_t)(num_pages - 1 - i)] = p;
        }
    } else {
        for (int32_t i = 0; i < num_pages; ++i) c->stack[(size_t)i] = num_pages - 1 - i;
    }
    *out = c;
    return SPKV_OK;
}

void spkv_cold_destroy(spkv_cold *cold) { delete cold; }

spkv_status spkv_seq_new(spkv_cold *c, int32_t *seq_out) {
    if (!c || !seq_out) return fail(SPKV_E_INVAL, "seq_new: null argument");
    c->seqs.emplace_back();
    c->live += 1;
    *seq_out = (int32_t)c->seqs.size() - 1;
    return SPKV_OK;
}

spkv_status spkv_cold_append_batch(spkv_cold *c, const int32_t *seqs, int32_t n, int32_t *slots_out,
                                   int32_t *cow_pairs_out, int32_t *n_cow_out, int32_t *n_done_out) {
    if (n_done_out) *n_done_out = 0;
    if (n_cow_out) *n_cow_out = 0;
    if (!c || n < 0 || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)) || !n_cow_out || !n_done_out)
        return fail(SPKV_E_INVAL, "append_batch: null argument or negative n");
    int32_t ncow = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t slot = 0, src = -1, dst = -1;
        spkv_status st = cold_append_one(c, seqs[i], &slot, &src, &dst);
        if (st != SPKV_OK) {
            *n_done_out = i;
            *n_cow_out = ncow;
            return st;
        }
        slots_out[i] = slot;
        if (src >= 0) {
            cow_pairs_out[2 * ncow] = src;
            cow_pairs_out[2 * ncow + 1] = dst;
            ++ncow;
        }
    }
    *n_done_out = n;
    *n_cow_out = ncow;
    return SPKV_OK;
}

spkv_status spkv_cold_fork(spkv_cold *c, int32_t src, int32_t *dst_out) {
    if (!c || !dst_out) return fail(SPKV_E_INVAL, "fork: null argument");
    spkv_cold::Seq *s = live_seq(c, src);
    if (!s) return fail(SPKV_E_STATE, "fork: unknown or released sequence " + std::to_string(src));
    spkv_cold::Seq child;
    child.table = s->table;
    child.len = s->len;
    for (int32_t pg : child.table) c->ref[pg] += 1;
    c->seqs.push_back(std::move(child));
    c->live += 1;
    *dst_out = (int32_t)c->seqs.size() - 1;
    return SPKV_OK;
}

spkv_status spkv_cold_release(spkv_cold *c, int32_t id) {
    if (!c) return fail(SPKV_E_INVAL, "release: null pool");
    spkv_cold::Seq *s = live_seq(c, id);
    if (!s) return fail(SPKV_E_STATE, "release: unknown or released sequence " + std::to_string(id));
    for (int32_t pg : s->table) {
        if (c->ref[pg] <= 0) return fail(SPKV_E_STATE, "release: page already free");
    }
    for (int32_t pg : s->table) {
        c->ref[pg] -= 1;
        if (c->ref[pg] == 0) c->stack.push_back(pg);
    }
    s->table.clear();
    s->len = 0;
    s->live = false;
    c->live -= 1;
    return SPKV_OK;
}

spkv_status spkv_cold_block_tables(const spkv_cold *c, const int32_t *seqs, int32_t n, int32_t max_blocks,
                                   int32_t *tables_out, int32_t *lens_out) {
    if (!c || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !lens_out || (max_blocks > 0 && !tables_out))))
        return fail(SPKV_E_INVAL, "block_tables: bad argument");
    for (int32_t i = 0; i < n; ++i) {
        const spkv_cold::Seq *s = live_seq(const_cast<spkv_cold *>(c), seqs[i]);
        if (!s) return fail(SPKV_E_STATE, "block_tables: unknown or released sequence");
        if ((int64_t)s->table.size() > max_blocks) return fail(SPKV_E_INVAL, "block_tables: table longer than max_blocks");
    }
    for (int32_t i = 0; i < n; ++i) {
        const spkv_cold::Seq &s = c->seqs[(size_t)seqs[i]];
        int32_t *row = tables_out + (int64_t)i * max_blocks;
        for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)s.table.size() ? s.table[(size_t)j] : -1;
        lens_out[i] = s.len;
    }
    return SPKV_OK;
}

spkv_status spkv_cold_get_info(const spkv_cold *c, spkv_cold_info *out) {
    if (!c || !out) return fail(SPKV_E_INVAL, "cold_get_info: null argument");
    out->num_pages = c->num_pages;
    out->page_size = c->page_size;
    out->num_free = (int32_t)c->stack.size();
    out->num_ids = (int32_t)c->seqs.size();
    out->num_live = c->live;
    return SPKV_OK;
}

spkv_status spkv_cold_refcounts(const spkv_cold *c, int32_t *ref_out) {
    if (!c || (!ref_out && c->num_pages > 0)) return fail(SPKV_E_INVAL, "cold_refcounts: null argument");
    std::copy(c->ref.begin(), c->ref.end(), ref_out);
    return SPKV_OK;
}

spkv_status spkv_cold_free_stack(const spkv_cold *c, int32_t *out) {
    if (!c || (!out && !c->stack.empty())) return fail(SPKV_E_INVAL, "cold_free_stack: null argument");
    std::copy(c->stack.begin(), c->stack.end(), out);
    return SPKV_OK;
}

spkv_status spkv_cold_seq_info(const spkv_cold *c, int32_t id, int32_t *len_out, int32_t *live_out,
                               int32_t *nblocks_out) {
    if (!c || !len_out || !live_out || !nblocks_out) return fail(SPKV_E_INVAL, "cold_seq_info: null argument");
    if (id < 0 || id >= (int32_t)c->seqs.size()) return fail(SPKV_E_STATE, "cold_seq_info: unknown id");
    const spkv_cold::Seq &s = c->seqs[(size_t)id];
    *len_out = s.len;
    *live_out = s.live ? 1 : 0;
    *nblocks_out = (int32_t)s.table.size();
    return SPKV_OK;
}

// =============================== HOT ========================================

spkv_status spkv_hot_create(int64_t capacity, spkv_hot **out) {
    if (!out || capacity < 0) return fail(SPKV_E_INVAL, "hot_create: bad argument");
    auto *h = new spkv_hot();
    h->capacity = capacity;
    if (capacity > 0) h->free.push_back({0, capacity});
    *out = h;
    return SPKV_OK;
}

void spkv_hot_destroy(spkv_hot *hot) { delete hot; }

spkv_status spkv_hot_alloc(spkv_hot *h, int64_t lp, int64_t *base_out) {
    if (!h || !base_out) return fail(SPKV_E_INVAL, "hot_alloc: null argument");
    if (lp <= 0) return fail(SPKV_E_INVAL, "hot_alloc: prefix length must be positive");
    std::vector<int64_t> order = lru_order(h);
    // Would evicting every unreferenced slab make room?  If not, change nothing.
    {
        auto fr = h->free;
        for (int64_t b : order) insert_range(fr, b, h->slabs.at(b).len);
        bool fits = false;
        for (auto &r : fr) fits = fits || r.second >= lp;
        if (!fits) return fail(SPKV_E_NOMEM, "HOT pool has no contiguous range of " + std::to_string(lp) + " tokens");
    }
    size_t next = 0;
    int64_t base;
    while (!first_fit(h->free, lp, &base)) {
        int64_t victim = order[next++];
        insert_range(h->free, victim, h->slabs.at(victim).len);
        h->slabs.erase(victim);
    }
    h->slabs[base] = spkv_hot::Slab{lp, 1, -1};
    *base_out = base;
    return SPKV_OK;
}

spkv_status spkv_hot_incref(spkv_hot *h, int64_t base) {
    if (!h) return fail(SPKV_E_INVAL, "hot_incref: null pool");
    auto it = h->slabs.find(base);
    if (it == h->slabs.end()) return fail(SPKV_E_STATE, "hot_incref: no slab at base " + std::to_string(base));
    it->second.ref += 1;
    it->second.lru = -1;
    return SPKV_OK;
}

spkv_status spkv_hot_decref(spkv_hot *h, int64_t base) {
    if (!h) return fail(SPKV_E_INVAL, "hot_decref: null pool");
    auto it = h->slabs.find(base);
    if (it == h->slabs.end()) return fail(SPKV_E_STATE, "hot_decref: no slab at base " + std::to_string(base));
    if (it->second.ref <= 0) return fail(SPKV_E_STATE, "hot_decref: slab is unreferenced");
    it->second.ref -= 1;
    if (it->second.ref == 0) it->second.lru = h->tick++;
    return SPKV_OK;
}

spkv_status spkv_hot_evict_unreferenced(spkv_hot *h, int32_t *n_evicted_out) {
    if (!h) return fail(SPKV_E_INVAL, "hot_evict: null pool");
    std::vector<int64_t> order = lru_order(h);
    for (int64_t b : order) {
        insert_range(h->free, b, h->slabs.at(b).len);
        h->slabs.erase(b);
    }
    if (n_evicted_out) *n_evicted_out = (int32_t)order.size();
    return SPKV_OK;
}

spkv_status spkv_hot_get_info(const spkv_hot *h, spkv_hot_info *out) {
    if (!h || !out) return fail(SPKV_E_INVAL, "hot_get_info: null argument");
    out->capacity = h->capacity;
    int64_t f = 0;
    for (auto &r : h->free) f += r.second;
    out->free_tokens = f;
    out->num_free_ranges = (int32_t)h->free.size();
    out->num_slabs = (int32_t)h->slabs.size();
    out->tick = h->tick;
    return SPKV_OK;
}

spkv_status spkv_hot_free_ranges(const spkv_hot *h, int64_t *base_out, int64_t *len_out, int32_t cap) {
    if (!h || cap < (int32_t)h->free.size() || (cap > 0 && (!base_out || !len_out)))
        return fail(SPKV_E_INVAL, "hot_free_ranges: bad argument or capacity too small");
    for (size_t i = 0; i < h->free.size(); ++i) {
        base_out[i] = h->free[i].first;
        len_out[i] = h->free[i].second;
    }
    return SPKV_OK;
}

spkv_status spkv_hot_slabs(const spkv_hot *h, int64_t *base_out, int64_t *len_out, int32_t *ref_out,
                           int64_t *lru_out, int32_t cap) {
    if (!h || cap < (int32_t)h->slabs.size() || (cap > 0 && (!base_out || !len_out || !ref_out || !lru_out)))
        return fail(SPKV_E_INVAL, "hot_slabs: bad argument or capacity too small");
    size_t i = 0;
    for (const auto &kv : h->slabs) {
        base_out[i] = kv.first;
        len_out[i] = kv.second.len;
        ref_out[i] = kv.second.ref;
        lru_out[i] = kv.second.lru;
        ++i;
    }
    return SPKV_OK;
}

}  // extern "C"
