// Internal declarations shared by the host runtime (C++) and the HIP launchers.
#pragma once

#include <cstdint>
#include <cstddef>
#include <string>
#include <vector>

#include "spkv.h"

#if defined(__HIPCC__)
#define SPKV_HD __host__ __device__
#else
#define SPKV_HD
#endif

namespace spkv {

// Thread-local error text behind spkv_last_error().
spkv_status fail(spkv_status code, const std::string &msg);
void clear_error();

// Limits of the library.
constexpr int kMaxGroups = 512;        // groups per step (cascade bitmask size)
constexpr int kMaxGqa = 8;             // Hq / Hkv
constexpr int kMaxKvHeads = 16;
constexpr int kFlatSplitCap = 64;      // partials per row from the flat pass
constexpr int kPrefixSplitCap = 64;    // partials per row from the prefix pass
constexpr int kPrefixKeyTile = 32;     // keys per MFMA tile in the prefix kernel
constexpr int kFlatWaves = 4;          // KV heads (one wave each) per flat block
constexpr int kFlatMinTokens = 64;     // shortest flat range per block
// Start cost of one (range, request) piece of the paged pass, in tokens: the
// ranges are cut with this many virtual tokens before each non-empty request,
// so a range that crosses request boundaries gets fewer real tokens (a new
// piece waits for its geometry, block-table and first ring fill).
constexpr int kFlatHeadTokens = 48;
constexpr int kFlatWaveSlots = 16;     // resident flat waves per CU (128 VGPRs), float32 pass
constexpr int kFlatMfmaTokens = 16;    // tokens per ring stage of the bf16 (MFMA) paged pass
constexpr int kFlatMfmaStages = 4;     // ring stages per wave of the bf16 paged pass
constexpr int kLdsPerCU = 160 * 1024;  // LDS bytes per CU (gfx950)
constexpr int kSplitPBelow = 256;      // prefixes shorter than this carry P as bf16 hi + lo

// Per-group cascade bitmask passed to kernels by value.
struct GroupMask {
    uint32_t bits[kMaxGroups / 32];
};

// One launch of the paged (flat) pass over a sub-batch of at most
// kFlatArgReqs requests.  Its tokens - every request's range of
// [HOT prefix ; COLD suffix] concatenated in request order - are cut into
// `blocks` equal ranges per group of up to kFlatWaves KV heads (stream-K), so
// every block carries the same work whatever the request lengths: the cut is
// made in virtual tokens, kFlatHeadTokens of them before each non-empty
// request, so each piece's start cost counts against its range.
// Passed by value as a kernel argument: blocks find their requests with a few
// scalar loads and no index pass.
constexpr int kFlatArgReqs = 256;
struct FlatLaunch {
    int32_t b0;                        // first request of the sub-batch
    int32_t nreq;                      // requests in it
    int32_t blocks;                    // ranges per head group (grid x)
    int32_t max_parts;                 // bound on partial states per request
    int64_t total;                     // virtual tokens of the sub-batch
    int32_t head;                      // virtual tokens before each non-empty request
    int32_t offs[kFlatArgReqs + 1];    // exclusive prefix sums of the virtual request lengths
                                       // (head + length, 0 for an empty request); request i's
                                       // tokens are [offs[i] + head, offs[i + 1])
};

// Range (block) index containing virtual token x when T are cut into nb
// ranges [floor(k*T/nb), floor((k+1)*T/nb)).
SPKV_HD inline int range_of(int64_t x, int64_t T, int nb) {
    int k = (int)((x * nb) / T);
    if (k + 1 < nb && (T * (k + 1)) / nb <= x) ++k;
    return k;
}

// Partial states written for request i of a flat launch, and its first range.
SPKV_HD inline int flat_parts(const FlatLaunch &f, int i, int *first) {
    const int64_t o0 = (int64_t)f.offs[i] + f.head, o1 = f.offs[i + 1];
    if (f.blocks <= 0 || o1 <= o0) {
        *first = 0;
        return 0;
    }
    const int k0 = range_of(o0, f.total, f.blocks);
    *first = k0;
    return range_of(o1 - 1, f.total, f.blocks) - k0 + 1;
}

// The launch plan of one decode call (host-computed, deterministic).
struct Plan {
    GroupMask cascade;        // bit g set: group g takes the prefix contraction
    int32_t num_groups;
    int32_t flat_chunk;       // virtual tokens per flat range (largest sub-batch)
    int32_t flat_splits;      // partial slots per row reserved for the flat pass
    int32_t prefix_chunk;     // base tau for the prefix pass (multiple of kPrefixKeyTile)
    int32_t prefix_splits;    // grid x of the prefix kernel
    int32_t prefix_waves;     // row waves per prefix block (32 rows each; float32: 1, a 256-thread block)
    int32_t prefix_key_halves;  // 2: each block's key chunk is split over two wave sets
    int32_t prefix_mtiles;    // grid y of the prefix kernel
    int32_t splits_total;     // prefix_splits + flat_splits (partial stride per row)
    int64_t flat_items;
    int64_t prefix_items;
    int64_t ws_bytes;
    std::vector<FlatLaunch> flat;    // paged pass (suffix, or whole context for flat-mode groups)
    int32_t flat_head_groups;        // grid y of the paged pass
    bool run_prefix;          // some cascade group has Lp > 0
    bool prefix_split_p;      // some cascade group is short: carry P as bf16 hi + lo
    bool single_launch;       // the paged pass and the prefix contraction may share one launch
    int64_t co_prefix_items;  // prefix items of cascade groups with a prefix (the co-resident launch's count)
    bool co_resident;         // single launch with both roles in every block: its prefix items fit beside
                              // the paged blocks in one round
    int32_t co_prefix_stages; // co-resident: prefix ring depth, 3 (paged rings of 3) or 5 (paged rings of 2)
};

// LDS bytes of one wave of the bf16 paged pass: its ring (K and V rows of
// kFlatMfmaTokens tokens per stage) and a 64-entry block-table buffer.
SPKV_HD constexpr int flat_mfma_wave_bytes(int d) { return kFlatMfmaStages * 2 * kFlatMfmaTokens * d * 2 + 256; }

// Resident paged-pass blocks per CU for blocks of `hpb` waves: the float32
// pass is bound by registers (kFlatWaveSlots waves), the bf16 pass by its
// LDS rings.
inline int flat_blocks_per_cu(bool bf16, int d, int hpb) {
    if (!bf16) return kFlatWaveSlots / hpb > 0 ? kFlatWaveSlots / hpb : 1;
    const int n = kLdsPerCU / (hpb * flat_mfma_wave_bytes(d));
    return n > 0 ? n : 1;
}

// Chunk length of one request or group: at least `tau`, large enough that at
// most `cap` chunks cover `len`, rounded up to `granule`.
SPKV_HD inline int32_t chunk_for(int64_t len, int32_t tau, int32_t cap, int32_t granule) {
    int64_t c = tau;
    int64_t need = (len + cap - 1) / cap;
    if (need > c) c = need;
    c = (c + granule - 1) / granule * granule;
    return (int32_t)c;
}
SPKV_HD inline int32_t splits_for(int64_t len, int32_t chunk) {
    return len <= 0 ? 0 : (int32_t)((len + chunk - 1) / chunk);
}

// Validate a batch descriptor and its pools (host side only; device arrays
// are not read).  kv may be null for plan-only calls.
spkv_status validate_batch(const spkv_batch *b, const spkv_kv *kv);

// Build the plan for a per-group choice (cascade[g] != 0 -> cascade; null -> all cascade).
spkv_status make_plan(const spkv_batch *b, const int32_t *cascade, int32_t num_cus, Plan *out);

// Compute units the split plan targets (MI355X: 256).  A constant, so plans
// and workspace sizes are the same with or without a device present.
constexpr int32_t kPlanCUs = 256;

// Upper bound of Plan::ws_bytes for any per-group choice.
size_t workspace_bound(const spkv_batch *b);

}  // namespace spkv
