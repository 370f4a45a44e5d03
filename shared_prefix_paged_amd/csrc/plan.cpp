// Host runtime: error state, batch validation, the per-call split plan and the
// per-step dispatcher.
//
// Split plan: the static partition of Tangram's Algorithm 1 (Section 4.3),
// applied to decode requests instead of head groups - a per-split budget
// tau = max(1, ceil(total / target_items)) and max(1, ceil(len / tau)) splits
// per request; here tau also has a floor (partial states cost traffic) and
// the splits per row are capped (workspace bound).  Partials of every split
// are combined by the log-sum-exp merge of the GraniKV paper's Eq. (1).
//
// Dispatcher: GraniKV paper, Section 3.6 - a thin per-step wrapper owning both
// backends over the same pools decides from the step's realized batch
// (M_eff = B_step * n_q/kv, its Eq. (2)) with a constant fitted to the GPU.
// Here the decision is cascade vs flat per prefix group, from a cost model
// whose constants are data.
#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "internal.h"

namespace spkv {

namespace {
thread_local std::string g_last_error;
}

spkv_status fail(spkv_status code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

void clear_error() { g_last_error.clear(); }

static int elem_bytes(int32_t dtype) { return dtype == SPKV_DTYPE_BF16 ? 2 : 4; }

spkv_status validate_batch(const spkv_batch *b, const spkv_kv *kv) {
    if (!b) return fail(SPKV_E_INVAL, "null batch");
    if (b->batch < 0) return fail(SPKV_E_INVAL, "negative batch");
    if (b->num_kv_heads < 1 || b->num_kv_heads > kMaxKvHeads) return fail(SPKV_E_INVAL, "num_kv_heads must be 1..16");
    if (b->num_q_heads < b->num_kv_heads || b->num_q_heads % b->num_kv_heads)
        return fail(SPKV_E_INVAL, "num_q_heads must be a multiple of num_kv_heads");
    if (b->num_q_heads / b->num_kv_heads > kMaxGqa) return fail(SPKV_E_INVAL, "GQA group size must be <= 8");
    if (b->head_dim != 64 && b->head_dim != 128) return fail(SPKV_E_INVAL, "head_dim must be 64 or 128");
    if (b->dtype != SPKV_DTYPE_BF16 && b->dtype != SPKV_DTYPE_F32) return fail(SPKV_E_INVAL, "unknown dtype");
    if (!std::isfinite(b->scale) || !(b->scale > 0.f)) return fail(SPKV_E_INVAL, "scale must be finite and positive");
    if (b->num_groups < 0 || b->num_groups > kMaxGroups) return fail(SPKV_E_INVAL, "num_groups must be 0..512");
    if (b->page_size < 1 || b->max_blocks < 0) return fail(SPKV_E_INVAL, "bad page_size/max_blocks");
    const int B = b->batch, ng = b->num_groups;
    if (B > 0 && (!b->q || !b->group_of || !b->cold_lens || !b->host_cold_lens || !b->host_group_of))
        return fail(SPKV_E_INVAL, "q, group_of, cold_lens and their host copies are required");
    if (B > 0 && b->max_blocks > 0 && !b->block_tables) return fail(SPKV_E_INVAL, "block_tables is required");
    if (ng > 0 && (!b->hot_base || !b->hot_len || !b->host_hot_base || !b->host_hot_len))
        return fail(SPKV_E_INVAL, "group arrays (device and host) are required when num_groups > 0");
    for (int g = 0; g < ng; ++g) {
        if (b->host_hot_len[g] < 0 || b->host_hot_base[g] < 0) return fail(SPKV_E_INVAL, "negative hot_base/hot_len");
        if ((int64_t)b->host_hot_len[g] * b->head_dim * 4 >= (int64_t(1) << 32))
            return fail(SPKV_E_INVAL, "group " + std::to_string(g) + " prefix longer than a 4 GiB slab per head");
        if (kv && b->host_hot_base[g] + b->host_hot_len[g] > kv->hot_capacity)
            return fail(SPKV_E_INVAL, "group " + std::to_string(g) + " slab exceeds the HOT capacity");
    }
    for (int i = 0; i < B; ++i) {
        if (b->host_group_of[i] < -1 || b->host_group_of[i] >= ng)
            return fail(SPKV_E_INVAL, "group_of[" + std::to_string(i) + "] outside [-1, num_groups)");
    }
    const int64_t cap_tokens = (int64_t)b->max_blocks * b->page_size;
    for (int i = 0; i < B; ++i) {
        if (b->host_cold_lens[i] < 0 || b->host_cold_lens[i] > cap_tokens)
            return fail(SPKV_E_INVAL, "cold_lens[" + std::to_string(i) + "] outside [0, max_blocks*page_size]");
    }
    if (kv) {
        if (kv->hot_capacity < 0 || kv->cold_slots < 0) return fail(SPKV_E_INVAL, "negative pool size");
        if (kv->num_layers < 1 || kv->layer < 0 || kv->layer >= kv->num_layers)
            return fail(SPKV_E_INVAL, "layer outside [0, num_layers) or num_layers < 1");
        if (kv->hot_capacity * b->num_kv_heads * kv->num_layers >= (int64_t(1) << 31) ||
            kv->cold_slots * b->num_kv_heads >= (int64_t(1) << 31))
            return fail(SPKV_E_INVAL, "pools limited to 2^31 rows (HOT: slots x KV heads x layers; COLD: per layer)");
        if (B > 0 && kv->cold_slots > 0 && (!kv->k_cold || !kv->v_cold)) return fail(SPKV_E_INVAL, "null COLD pool");
        if (ng > 0 && kv->hot_capacity > 0 && (!kv->k_hot || !kv->v_hot)) return fail(SPKV_E_INVAL, "null HOT pool");
        if (kv->cold_slots % b->page_size) return fail(SPKV_E_INVAL, "cold_slots must be a multiple of page_size");
    }
    return SPKV_OK;
}

static inline bool mask_get(const GroupMask &m, int g) { return (m.bits[g >> 5] >> (g & 31)) & 1u; }

// Requests per group ([GKV] Section 3.4: a request belongs to the group whose
// prefix it shares), counted from group_of; validated batches only.
static std::vector<int64_t> member_counts(const spkv_batch *b) {
    std::vector<int64_t> n((size_t)std::max(0, b->num_groups), 0);
    for (int i = 0; i < b->batch; ++i)
        if (b->host_group_of[i] >= 0) n[(size_t)b->host_group_of[i]] += 1;
    return n;
}

// Stream-K launches of one paged pass over per-request lengths L (sub-batches
// of at most kFlatArgReqs requests).  Each launch gets as many equal ranges of
// virtual tokens (kFlatHeadTokens before each non-empty request, then its
// tokens) per head group as one full round of resident blocks, no more than
// one per kFlatMinTokens real tokens, and few enough that no request spans
// more than kFlatSplitCap ranges.
static std::vector<FlatLaunch> plan_flat(const std::vector<int64_t> &L, int head_groups, int blocks_per_cu,
                                         int32_t num_cus) {
    std::vector<FlatLaunch> out;
    const int B = (int)L.size();
    const int64_t resident = std::max<int64_t>(1, (int64_t)num_cus * blocks_per_cu / head_groups);
    for (int b0 = 0; b0 < B; b0 += kFlatArgReqs) {
        FlatLaunch f{};
        f.b0 = b0;
        f.nreq = std::min(kFlatArgReqs, B - b0);
        int64_t T = 0, max_len = 0, real = 0;
        f.head = kFlatHeadTokens;
        for (int i = 0; i < f.nreq; ++i) {
            f.offs[i] = (int32_t)T;
            const int64_t l = L[(size_t)(b0 + i)];
            T += l > 0 ? l + f.head : 0;
            real += l;
            max_len = std::max<int64_t>(max_len, l);
        }
        f.offs[f.nreq] = (int32_t)T;
        f.total = T;
        if (T == 0) {            // kept (blocks = 0) so sub-batch i is entry i of every pass
            out.push_back(f);
            continue;
        }
        int64_t nb = std::min<int64_t>(resident, (real + kFlatMinTokens - 1) / kFlatMinTokens);
        nb = std::max<int64_t>(nb, 1);
        auto parts = [&](int64_t n) { return (max_len + T / n - 1) / (T / n) + 1; };
        while (nb > 1 && parts(nb) > kFlatSplitCap) nb = std::max<int64_t>(1, nb * 3 / 4);
        f.blocks = (int32_t)nb;
        f.max_parts = (int32_t)std::min<int64_t>(kFlatSplitCap, parts(nb));
        out.push_back(f);
    }
    return out;
}

spkv_status make_plan(const spkv_batch *b, const int32_t *cascade, int32_t num_cus, Plan *p) {
    *p = Plan{};
    p->prefix_key_halves = 1;
    const int B = b->batch, ng = b->num_groups, Hkv = b->num_kv_heads, D = b->head_dim;
    const int G = b->num_q_heads / Hkv;
    p->num_groups = ng;
    for (int g = 0; g < ng; ++g)
        if (!cascade || cascade[g]) p->cascade.bits[g >> 5] |= 1u << (g & 31);

    const bool bf16 = b->dtype == SPKV_DTYPE_BF16;
    const std::vector<int64_t> members = member_counts(b);
    int64_t prefix_work = 0;        // row tiles x keys of the MFMA prefix pass
    int64_t max_m = 0, max_lp_c = 0;
    for (int g = 0; g < ng; ++g) {
        const int64_t n = members[(size_t)g];
        const int64_t lp = b->host_hot_len[g];
        if (n == 0 || lp == 0 || !mask_get(p->cascade, g)) continue;
        max_m = std::max<int64_t>(max_m, n * G);
        max_lp_c = std::max<int64_t>(max_lp_c, lp);
        if (lp < kSplitPBelow) p->prefix_split_p = true;
    }

    // ---- flat pass (stream-K over each sub-batch's concatenated tokens) -----
    const int hpb = std::min(Hkv, kFlatWaves);
    p->flat_head_groups = (Hkv + hpb - 1) / hpb;
    {
        std::vector<int64_t> L((size_t)B);
        for (int i = 0; i < B; ++i) {
            const int g = b->host_group_of[i];
            const bool dense_member = g >= 0 && !mask_get(p->cascade, g);
            L[(size_t)i] = b->host_cold_lens[i] + (dense_member ? b->host_hot_len[g] : 0);
        }
        p->flat = plan_flat(L, p->flat_head_groups, flat_blocks_per_cu(bf16, D, hpb), num_cus);
    }
    for (const auto &f : p->flat)
        if (f.total >= (int64_t(1) << 31)) return fail(SPKV_E_INVAL, "a paged-pass sub-batch exceeds 2^31 tokens");
    p->flat_splits = 0;
    p->flat_chunk = 0;
    for (const auto &f : p->flat) {
        p->flat_splits = std::max(p->flat_splits, f.max_parts);
        if (f.blocks > 0) p->flat_chunk = std::max<int32_t>(p->flat_chunk, (int32_t)(f.total / f.blocks));
    }
    // Whether the paged pass's blocks fit one launch with prefix blocks
    // (paged_prefix_kernel): one sub-batch at d = 128 whose blocks of hpb
    // KV-head waves (hpb = 1, 2 or 4) fill a CU's LDS 4 / hpb at a time, as
    // the paged plan counts them.
    const bool paged_one_launch = bf16 && D == 128 && p->flat.size() == 1 && p->flat[0].blocks > 0 &&
                                  kFlatWaves % hpb == 0 && flat_blocks_per_cu(bf16, D, hpb) == kFlatWaves / hpb;

    // ---- prefix pass ------------------------------------------------------
    // One batched contraction per cascade group and KV head in both dtypes:
    // bf16 on MFMA in row tiles of 1, 2 or 4 waves of 32 rows; float32 on the
    // VALU in row tiles of 32 rows.  Same key-split rule for both.
    p->run_prefix = max_lp_c > 0;
    if (p->run_prefix) {
        int w = (int)std::min<int64_t>(4, (max_m + 31) / 32);
        p->prefix_waves = !bf16 ? 1 : (w <= 1 ? 1 : (w == 2 ? 2 : 4));   // bf16 tile variants: 1, 2 or 4 waves
        // Tiles of 4 row waves take the two-key-half variant: one 8-wave block
        // (two 64 KB rings) per CU instead of two 4-wave blocks, and half as
        // many partial states per row.  Tiles of 2 row waves take it only where
        // the paged pass and the prefix contraction then share one launch: on
        // its own that tile ran slower than two 2-wave blocks of one half
        // (C4: 71.7 against 64 us), in the one launch the pair is faster.
        p->prefix_key_halves =
            p->prefix_waves == 4 || (p->prefix_waves == 2 && paged_one_launch && !p->prefix_split_p) ? 2 : 1;
        const int64_t mt = 32 * p->prefix_waves;
        p->prefix_mtiles = (int32_t)((max_m + mt - 1) / mt);
        for (int g = 0; g < ng; ++g) {
            const int64_t n = members[(size_t)g];
            const int64_t lp = b->host_hot_len[g];
            if (n == 0 || lp == 0 || !mask_get(p->cascade, g)) continue;
            prefix_work += Hkv * ((n * G + mt - 1) / mt) * lp;
        }
        // 128 KB of LDS rings per CU: two blocks of one key half or one block
        // of two.  Size the key chunk so that all blocks fit in one round.
        // Rounding each group's last chunk up can add a block per row tile,
        // so grow the chunk until the exact block count fits (or every group
        // is one chunk).
        const int64_t target = std::max<int64_t>(1, (int64_t)num_cus * 2 / p->prefix_key_halves);
        int64_t pt = (prefix_work + target - 1) / target;
        // A floor on the chunk keeps partial states (written, then merged) few
        // per row; the float32 contraction works a tile at a time and takes a
        // lower one so short prefixes still spread over several blocks.
        pt = std::max<int64_t>(pt, bf16 ? 256 : 64);
        pt = (pt + kPrefixKeyTile - 1) / kPrefixKeyTile * kPrefixKeyTile;
        auto blocks_for = [&](int64_t chunk) {
            int64_t nb = 0;
            for (int g = 0; g < ng; ++g) {
                const int64_t n = members[(size_t)g];
                const int64_t lp = b->host_hot_len[g];
                if (n == 0 || lp == 0 || !mask_get(p->cascade, g)) continue;
                nb += Hkv * ((n * G + mt - 1) / mt) *
                      splits_for(lp, chunk_for(lp, (int32_t)chunk, kPrefixSplitCap, kPrefixKeyTile));
            }
            return nb;
        };
        while (pt < max_lp_c && pt < (1 << 20) && blocks_for(pt) > target) pt += kPrefixKeyTile;
        p->prefix_chunk = (int32_t)std::min<int64_t>(pt, 1 << 20);
        p->prefix_splits = std::min<int32_t>(kPrefixSplitCap, splits_for(max_lp_c, p->prefix_chunk));
    }
    p->splits_total = p->prefix_splits + p->flat_splits;
    // One launch for both passes (paged_prefix_kernel) where its blocks keep
    // the shapes the two plans assume: the paged blocks above, and prefix
    // tiles of 2 or 4 row waves with two key halves (one block per CU).
    p->single_launch = paged_one_launch && p->run_prefix && p->prefix_waves >= 2 && p->prefix_key_halves == 2 &&
                       !p->prefix_split_p;

    // Prefix items as the co-resident launch numbers them: every cascade group
    // with a prefix, members or not, at the plan's row tiles.
    p->co_prefix_items = 0;
    if (p->run_prefix)
        for (int g = 0; g < ng; ++g) {
            const int64_t lp = b->host_hot_len[g];
            if (lp <= 0 || !mask_get(p->cascade, g)) continue;
            p->co_prefix_items += (int64_t)Hkv * p->prefix_mtiles *
                                  splits_for(lp, chunk_for(lp, p->prefix_chunk, kPrefixSplitCap, kPrefixKeyTile));
        }

    {
        const int per = kFlatWaves / hpb;
        const int64_t paged_blocks =
            p->flat.empty() ? 0 : ((int64_t)p->flat[0].blocks * p->flat_head_groups + per - 1) / per;
        p->co_resident = p->single_launch && p->co_prefix_items <= paged_blocks;
    }
    // Ring depths of the co-resident launch.  Each role's share of the memory
    // bandwidth follows the bytes it keeps in flight; the deeper prefix ring
    // (and shallower paged rings) pays where the prefix items' key tiles
    // outnumber the ring stages of a paged wave's range, i.e. where the
    // prefix role would otherwise finish last.
    p->co_prefix_stages = 0;
    if (p->co_resident) {
        const int64_t item_tiles = (std::min<int64_t>(max_lp_c, chunk_for(max_lp_c, p->prefix_chunk, kPrefixSplitCap,
                                                                          kPrefixKeyTile)) +
                                    kPrefixKeyTile - 1) / kPrefixKeyTile;
        const int64_t paged_stages = (p->flat_chunk + kFlatMfmaTokens - 1) / kFlatMfmaTokens;
        p->co_prefix_stages = p->prefix_waves == 4 && item_tiles > paged_stages ? 5 : 3;
    }

    // Item counts (informational).
    p->flat_items = 0;
    p->prefix_items = 0;
    for (const auto &f : p->flat) p->flat_items += (int64_t)f.blocks * p->flat_head_groups;
    for (int g = 0; g < ng; ++g) {
        const int64_t n = members[(size_t)g];
        const int64_t lp = b->host_hot_len[g];
        if (n == 0 || lp == 0) continue;
        if (mask_get(p->cascade, g)) {
            {
                const int64_t mt = 32 * p->prefix_waves;
                p->prefix_items += Hkv * ((n * G + mt - 1) / mt) *
                                   splits_for(lp, chunk_for(lp, p->prefix_chunk, kPrefixSplitCap, kPrefixKeyTile));
            }
        }
    }
    const int64_t rows = (int64_t)B * b->num_q_heads;
    p->ws_bytes = rows * p->splits_total * (int64_t)(D + 1) * 4 + 256;
    (void)elem_bytes;
    return SPKV_OK;
}

size_t workspace_bound(const spkv_batch *b) {
    const int64_t rows = (int64_t)b->batch * b->num_q_heads;
    return (size_t)(rows * (kPrefixSplitCap + kFlatSplitCap) * (int64_t)(b->head_dim + 1) * 4 + 256);
}

}  // namespace spkv

using namespace spkv;

extern "C" {

const char *spkv_last_error(void) {
    static thread_local std::string copy;
    copy = spkv::g_last_error;
    return copy.c_str();
}

const char *spkv_version(void) { return "spkv 0.1 (gfx950)"; }

size_t spkv_workspace_size(const spkv_batch *batch) {
    if (validate_batch(batch, nullptr) != SPKV_OK) return 0;
    return workspace_bound(batch);
}

spkv_status spkv_plan_query(const spkv_batch *batch, const int32_t *cascade, spkv_plan_info *out) {
    if (!out) return fail(SPKV_E_INVAL, "plan_query: null out");
    spkv_status st = validate_batch(batch, nullptr);
    if (st != SPKV_OK) return st;
    Plan p;
    st = make_plan(batch, cascade, kPlanCUs, &p);
    if (st != SPKV_OK) return st;
    out->flat_chunk = p.flat_chunk;
    out->flat_splits = p.flat_splits;
    out->prefix_chunk = p.prefix_chunk;
    out->prefix_splits = p.prefix_splits;
    out->prefix_waves = p.prefix_waves;
    out->prefix_mtiles = p.prefix_mtiles;
    out->flat_items = p.flat_items;
    out->prefix_items = p.prefix_items;
    out->workspace_bytes = p.ws_bytes;
    out->flat_split_cap = kFlatSplitCap;
    out->flat_head_tokens = kFlatHeadTokens;
    out->prefix_split_cap = kPrefixSplitCap;
    out->prefix_granule = kPrefixKeyTile;
    out->prefix_key_halves = p.prefix_key_halves;
    out->single_launch = p.single_launch ? 1 : 0;
    out->co_resident = p.co_resident ? 1 : 0;
    out->co_prefix_stages = p.co_prefix_stages;
    return SPKV_OK;
}

spkv_status spkv_plan_parts(const spkv_batch *batch, const int32_t *cascade, int32_t *flat_parts_out,
                            int32_t *prefix_parts_out) {
    spkv_status st = validate_batch(batch, nullptr);
    if (st != SPKV_OK) return st;
    Plan p;
    st = make_plan(batch, cascade, kPlanCUs, &p);
    if (st != SPKV_OK) return st;
    const int B = batch->batch;
    int first = 0;
    if (flat_parts_out) {
        for (int b = 0; b < B; ++b) flat_parts_out[b] = 0;
        for (const auto &f : p.flat)
            for (int i = 0; i < f.nreq; ++i) flat_parts_out[f.b0 + i] = flat_parts(f, i, &first);
    }
    if (prefix_parts_out) {
        for (int b = 0; b < B; ++b) prefix_parts_out[b] = 0;
        if (p.run_prefix) {
            for (int b = 0; b < B; ++b) {
                const int g = batch->host_group_of[b];
                if (g < 0 || !((p.cascade.bits[g >> 5] >> (g & 31)) & 1u)) continue;
                const int64_t lp = batch->host_hot_len[g];
                if (lp <= 0) continue;
                prefix_parts_out[b] = std::min<int32_t>(
                    p.prefix_splits, splits_for(lp, chunk_for(lp, p.prefix_chunk, kPrefixSplitCap, kPrefixKeyTile)));
            }
        }
    }
    return SPKV_OK;
}

void spkv_dispatch_params_default(spkv_dispatch_params *p) {
    if (!p) return;
    // Fitted on MI355X to the cascade-vs-flat sweeps of the 8B-shaped (Hq 32,
    // Hkv 8) and 32B-shaped (Hq 10, Hkv 2) layers: prefix length 64 .. 32768
    // at 64 and 256 requests, and 1 .. 256 requests sharing a 4096- or
    // 16384-token prefix.  The flat pass re-reads a shared prefix at ~10 TB/s
    // (the re-reads are mostly cache hits); the cascade path costs ~7.5 us per
    // step (the prefix items beside the paged blocks in the co-resident launch,
    // and the merge's share) plus ~2 ns per query row of the groups that take
    // it (their partial states, written and merged).  With 2 ns per row, any
    // fixed cost in [7.0, 8.0] us picks the faster backend at every swept
    // point whose two times differ by more than 1 us (51 of the 52; the other
    // differs by 0.3 us).  The prefix contraction's own rates matter little
    // near the crossover; they are those of the kernel at the 8B shape.
    p->mode = SPKV_MODE_PER_GROUP;
    p->min_group_requests = 2;
    p->fixed_cost_us = 7.5;
    p->flat_gbps = 10000.0;
    p->prefix_gbps = 4000.0;
    p->prefix_tflops = 420.0;
    p->row_cost_ns = 2.0;
    p->single_launch = 1;
}

spkv_status spkv_dispatch(const spkv_batch *b, const spkv_dispatch_params *prm, int32_t *cascade_out) {
    spkv_status st = validate_batch(b, nullptr);
    if (st != SPKV_OK) return st;
    if (!prm || (b->num_groups > 0 && !cascade_out)) return fail(SPKV_E_INVAL, "dispatch: null argument");
    const int ng = b->num_groups;
    const int G = b->num_q_heads / b->num_kv_heads;
    const double kvb = 2.0 * b->num_kv_heads * b->head_dim * elem_bytes(b->dtype);
    switch (prm->mode) {
    case SPKV_MODE_FORCE_CASCADE:
        for (int g = 0; g < ng; ++g) cascade_out[g] = 1;
        return SPKV_OK;
    case SPKV_MODE_FORCE_DENSE:
        for (int g = 0; g < ng; ++g) cascade_out[g] = 0;
        return SPKV_OK;
    case SPKV_MODE_BATCH_GLOBAL: {
        // One batch-wide shared level: only when every request shares group 0's prefix.
        const bool all_one = ng == 1 && b->batch > 0 && member_counts(b)[0] == b->batch;
        for (int g = 0; g < ng; ++g) cascade_out[g] = all_one ? 1 : 0;
        return SPKV_OK;
    }
    case SPKV_MODE_PER_GROUP:
        break;
    default:
        return fail(SPKV_E_INVAL, "dispatch: unknown mode");
    }
    if (prm->flat_gbps <= 0 || prm->prefix_gbps <= 0 || prm->prefix_tflops <= 0)
        return fail(SPKV_E_INVAL, "dispatch: rates must be positive");
    if (prm->row_cost_ns < 0) return fail(SPKV_E_INVAL, "dispatch: negative row cost");
    // A group's benefit from cascade is the time the flat pass spends re-reading
    // its prefix for every member, minus its prefix contraction and the cost of
    // its query rows' extra partial states.  The fixed cost is paid once per
    // step by whichever groups take cascade, so the set of groups with a
    // positive benefit goes cascade exactly when their total benefit exceeds it
    // (this minimises the modelled step time).
    const std::vector<int64_t> members = member_counts(b);
    double total = 0.0;
    for (int g = 0; g < ng; ++g) {
        cascade_out[g] = 0;
        const int64_t n = members[(size_t)g];
        const double lp = (double)b->host_hot_len[g];
        if (n < prm->min_group_requests || lp <= 0 || b->dtype != SPKV_DTYPE_BF16) continue;
        // Effective M of the group's prefix contraction (Eq. (2) per group).
        const double m_eff = (double)n * G;
        const double t_flat = n * lp * kvb / (prm->flat_gbps * 1e3);                    // us
        const double t_bytes = lp * kvb / (prm->prefix_gbps * 1e3);
        const double t_flops = 4.0 * m_eff * lp * b->head_dim * b->num_kv_heads / (prm->prefix_tflops * 1e6);
        const double t_rows = prm->row_cost_ns * (double)n * b->num_q_heads * 1e-3;
        const double benefit = t_flat - std::max(t_bytes, t_flops) - t_rows;
        if (benefit > 0.0) {
            cascade_out[g] = 1;
            total += benefit;
        }
    }
    if (total <= prm->fixed_cost_us)
        for (int g = 0; g < ng; ++g) cascade_out[g] = 0;
    return SPKV_OK;
}

}  // extern "C"
