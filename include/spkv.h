/*
 * spkv.h - HOT/COLD KV cache and decode attention for AMD MI355X (gfx950).
 *
 * C ABI of libspkv.so.  Plain pointers and sizes only.
 *
 * Method sources:
 *   [GKV]  "GraniKV: Asymmetric Granularity KV-Cache Paging for Multi-Agent
 *          Systems with Long Shared Prefix" (paper deep-dive page).
 *   [PKV]  "Paged KV cache" (deep-dive page: How it works, Code,
 *          Implementation notes).
 *   [TGM]  "Tangram: Unlocking Non-Uniform KV Cache for Efficient Multi-turn
 *          LLM Serving", Section 4.3 and Algorithm 1 (static split plan).
 *
 * Conventions
 *   - Every call returns spkv_status.  SPKV_OK (0) on success, a negative code
 *     otherwise; spkv_last_error() then describes the failure (thread-local,
 *     valid until the next failing call on the same thread).  No C++
 *     exception crosses this interface.
 *   - A failing call leaves every allocator object exactly as it was (batch
 *     calls: the prefix of the batch that completed stays applied, and the
 *     count of completed items is reported).
 *   - Host allocator handles are owned by the caller (create/destroy), are
 *     single-owner and not thread-safe.
 *   - All device memory is allocated and owned by the caller.  Device-op
 *     calls only enqueue work on the given stream (a hipStream_t passed as
 *     void*; NULL is the null stream) and return before it runs.  They never
 *     allocate device memory: scratch space is the caller's workspace.
 *   - Layouts (row-major, element type per `dtype`):
 *       Q        [B, Hq, d]
 *       HOT      per pool of L layers: [capacity_tokens * L * Hkv * d]; a
 *                prefix of length Lp admitted at token slot `base` keeps
 *                head h of layer l as one dense [Lp, d] matrix starting at
 *                row base*Hkv*L + l*Lp*Hkv + h*Lp ([GKV] Section 3.2 stride:
 *                the slab holds all L layers of the prefix, layer-major).
 *       COLD     per pool of L layers: [L, num_pages * page_size, Hkv, d]
 *                (layer-major; every layer uses the same slots and block
 *                tables); token t of a sequence lives at slot
 *                table[t / P] * P + t % P ([PKV] How it works).
 *                One layer's COLD pool starts at element
 *                layer * num_pages * page_size * Hkv * d.
 *       out      [B, Hq, d] float32 (normalised attention output)
 *       lse      [B, Hq] float32, natural-log log-sum-exp of the scaled scores
 *   - GQA: query head j reads KV head j / (Hq / Hkv).
 */
#ifndef SPKV_H
#define SPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t spkv_status;
#define SPKV_OK        0
#define SPKV_E_INVAL  (-1)   /* bad argument, shape, dtype or size */
#define SPKV_E_NOMEM  (-2)   /* pool exhausted; state unchanged ([PKV] Code: alloc returns None) */
#define SPKV_E_STATE  (-3)   /* double release, decref of a free block, unknown id */
#define SPKV_E_HIP    (-4)   /* a HIP runtime call failed (launch, copy, device query) */

#define SPKV_DTYPE_BF16 0
#define SPKV_DTYPE_F32  1

/* Thread-local description of the last failure on this thread ("" if none). */
const char *spkv_last_error(void);
/* Library version string. */
const char *spkv_version(void);

/* ======================================================================
 * HOT pool: contiguous slabs for shared prefixes ([GKV] Section 3.2).
 * First-fit over address-ordered free ranges; a slab whose refcount drops to
 * zero stays resident and can be revived by spkv_hot_incref until it is
 * evicted.  Eviction is least-recently-released first and merges the freed
 * range with its free neighbours.
 * ==================================================================== */
typedef struct spkv_hot spkv_hot;

/* capacity_tokens >= 0.  *out receives a new handle. */
spkv_status spkv_hot_create(int64_t capacity_tokens, spkv_hot **out);
void        spkv_hot_destroy(spkv_hot *hot);

/* Reserve lp > 0 contiguous token slots; *base_out = first slot.  The slab
 * starts with refcount 1.  If no free range fits, unreferenced slabs are
 * evicted (oldest release first, one at a time, first-fit retried after each)
 * but only when evicting all of them would make room.  Otherwise returns
 * SPKV_E_NOMEM and nothing changes: the caller stores that prefix in the COLD
 * pool instead ([GKV] Appendix B.10). */
spkv_status spkv_hot_alloc(spkv_hot *hot, int64_t lp, int64_t *base_out);
/* Add / drop one reference to the slab at `base` (SPKV_E_STATE if there is no
 * slab there, or on decref of an unreferenced slab). */
spkv_status spkv_hot_incref(spkv_hot *hot, int64_t base);
spkv_status spkv_hot_decref(spkv_hot *hot, int64_t base);
/* Evict every unreferenced slab; *n_evicted_out may be NULL. */
spkv_status spkv_hot_evict_unreferenced(spkv_hot *hot, int32_t *n_evicted_out);

typedef struct spkv_hot_info {
    int64_t capacity;          /* tokens */
    int64_t free_tokens;       /* sum of free-range lengths */
    int32_t num_free_ranges;
    int32_t num_slabs;         /* resident slabs, referenced or not */
    int64_t tick;              /* release counter used for LRU order */
} spkv_hot_info;
spkv_status spkv_hot_get_info(const spkv_hot *hot, spkv_hot_info *out);
/* Free ranges in ascending base order; arrays hold `cap` entries. */
spkv_status spkv_hot_free_ranges(const spkv_hot *hot, int64_t *base_out, int64_t *len_out, int32_t cap);
/* Resident slabs in ascending base order; lru_out[i] = -1 while referenced,
 * else the release tick.  Arrays hold `cap` entries. */
spkv_status spkv_hot_slabs(const spkv_hot *hot, int64_t *base_out, int64_t *len_out,
                           int32_t *ref_out, int64_t *lru_out, int32_t cap);

/* ======================================================================
 * COLD pool: pages of `page_size` token slots with refcounts, a LIFO free
 * stack, copy-on-write and fork ([PKV] How it works, Code; [GKV] Section 3.3
 * uses page size 1).
 * ==================================================================== */
typedef struct spkv_cold spkv_cold;

/* num_pages >= 0, page_size >= 1.  free_order (nullable, num_pages entries,
 * a permutation of 0..num_pages-1) is the order in which pages are handed
 * out; NULL means 0, 1, 2, ... */
spkv_status spkv_cold_create(int32_t num_pages, int32_t page_size, const int32_t *free_order,
                             spkv_cold **out);
void        spkv_cold_destroy(spkv_cold *cold);

/* New empty sequence; ids are issued 0, 1, 2, ... and never reused. */
spkv_status spkv_seq_new(spkv_cold *cold, int32_t *seq_out);

/* For i in 0..n-1, in array order, give token number len of seqs[i] its
 * slot ([PKV] How it works and Code: append with copy-on-write).  That token
 * belongs to page len / P of the sequence, at row len % P.  A sequence only
 * writes into a page it holds alone, so a page is taken from the free stack
 * when the token starts a new page, or when its page is still shared with
 * another sequence after a fork; in the second case the shared page loses one
 * reference, the new page replaces it in the table and (old, new) is reported
 * as a copy-on-write pair (the caller copies the page before writing).
 * slots_out[n] receives the slots; cow_pairs_out[2*k], [2*k+1] the k-th
 * (src, dst) pair (at most n pairs), *n_cow_out their count, *n_done_out the
 * appends that completed.  Stops at the first failure (SPKV_E_NOMEM or
 * SPKV_E_STATE), leaving that append and the rest undone. */
spkv_status spkv_cold_append_batch(spkv_cold *cold, const int32_t *seqs, int32_t n, int32_t *slots_out,
                                   int32_t *cow_pairs_out, int32_t *n_cow_out, int32_t *n_done_out);
/* New sequence sharing every page of src (refcount + 1 each); nothing is
 * copied ([PKV] Code, fork). */
spkv_status spkv_cold_fork(spkv_cold *cold, int32_t src_seq, int32_t *dst_seq_out);
/* Drop one reference to every page of seq in table order and retire the id
 * ([PKV] Code, release).  A second release is SPKV_E_STATE. */
spkv_status spkv_cold_release(spkv_cold *cold, int32_t seq);
/* Block tables of n sequences as an [n, max_blocks] int32 array padded with
 * -1, plus their lengths.  SPKV_E_INVAL if a table is longer than max_blocks. */
spkv_status spkv_cold_block_tables(const spkv_cold *cold, const int32_t *seqs, int32_t n, int32_t max_blocks,
                                   int32_t *tables_out, int32_t *lens_out);

typedef struct spkv_cold_info {
    int32_t num_pages;
    int32_t page_size;
    int32_t num_free;
    int32_t num_ids;           /* ids issued so far */
    int32_t num_live;          /* ids not yet released */
} spkv_cold_info;
spkv_status spkv_cold_get_info(const spkv_cold *cold, spkv_cold_info *out);
/* Per-page refcounts, num_pages entries. */
spkv_status spkv_cold_refcounts(const spkv_cold *cold, int32_t *ref_out);
/* Free stack bottom -> top (the top is handed out next), num_free entries. */
spkv_status spkv_cold_free_stack(const spkv_cold *cold, int32_t *out);
/* Length, liveness and page count of one sequence id. */
spkv_status spkv_cold_seq_info(const spkv_cold *cold, int32_t seq, int32_t *len_out, int32_t *live_out,
                               int32_t *num_blocks_out);

/* ======================================================================
 * Cache writes (device, stream-ordered).
 * ==================================================================== */

/* Store layer `layer` of a prefix's K and V, each [lp, Hkv, d] token-major,
 * into its HOT slab at `base` in a pool of num_layers layers: element
 * (t, h, c) goes to ((base*Hkv*L + layer*lp*Hkv + h*lp) + t)*d + c ([GKV]
 * Section 3.2).  SPKV_E_INVAL unless 0 <= base, base+lp <= capacity and
 * 0 <= layer < num_layers. */
spkv_status spkv_hot_write(const void *k_src, const void *v_src, int64_t base, int64_t lp,
                           void *k_hot, void *v_hot, int64_t hot_capacity, int32_t num_layers, int32_t layer,
                           int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void *stream);

/* Write token i's K and V rows ([n, Hkv, d] each) at COLD slot
 * slot_mapping[i] ([PKV] How it works, step 1: reshape_and_cache).
 * k_cold / v_cold are one layer's pool (for layer l of a multi-layer pool,
 * the pool pointer plus l * cold_slots * Hkv * d elements).  slot_mapping is
 * device memory.  Slots outside [0, cold_slots) (e.g. -1 padding) are
 * skipped. */
spkv_status spkv_reshape_and_cache(const void *k_new, const void *v_new, const int32_t *slot_mapping,
                                   int32_t n, void *k_cold, void *v_cold, int64_t cold_slots,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void *stream);

/* Copy-on-write page copies ([PKV] How it works, step 2): for each of the n
 * (src, dst) pairs in device memory `pairs` ([n, 2] int32), copy all
 * page_size slots of page src to page dst, K and V, in every one of the
 * num_layers layers of the pool (a page is shared or copied for all layers
 * at once).  Pairs with a page outside [0, num_pages) are skipped.
 * Destination pages must be distinct and must not be the source of another
 * pair (true of pairs from append). */
spkv_status spkv_copy_blocks(const int32_t *pairs, int32_t n, void *k_cold, void *v_cold,
                             int32_t num_pages, int32_t page_size, int32_t num_layers,
                             int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void *stream);

/* One decode step's appends in one launch ([PKV] How it works, steps 1-3):
 * token i's K and V rows ([n, Hkv, d] each, device) are written at COLD slot
 * host_slots[i], and, when tables is not NULL, request r = host_rows[i] (or i
 * when host_rows is NULL) gets
 *     tables[r * max_blocks + lens[r] / P] = host_slots[i] / P;  lens[r] += 1
 * on the device (a fresh page, a copy-on-write replacement or an append into
 * the current page alike).  host_slots and host_rows are host arrays (the
 * allocator's output); their values are copied into the launch at call time,
 * so no upload is needed.  Rows must be distinct within one call.  Returns
 * SPKV_E_INVAL, before anything is launched, for a slot outside
 * [0, cold_slots) or (with tables) a row outside [0, num_rows); a block-table
 * entry that would land beyond max_blocks (a device length, not checked on
 * the host) is skipped.  Run spkv_copy_blocks for the step's copy-on-write
 * pairs first: the copy must not overwrite the new token. */
spkv_status spkv_append_tokens(const void *k_new, const void *v_new, const int32_t *host_slots,
                               const int32_t *host_rows, int32_t n, void *k_cold, void *v_cold, int64_t cold_slots,
                               int32_t *tables, int32_t max_blocks, int32_t *lens, int32_t num_rows,
                               int32_t page_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                               void *stream);

/* Device-side mirror of one append per request ([PKV] How it works, steps 2
 * and 3: the new token's page enters the block table the attention kernel
 * reads).  For i in 0..n-1 with r = rows[i]:
 *     tables[r * max_blocks + lens[r] / P] = slots[i] / P;  lens[r] += 1
 * which covers a fresh page, a copy-on-write replacement and an append into
 * the current page alike.  tables, lens, rows and slots are device memory;
 * rows must be distinct within one call.  Rows outside [0, num_rows) and
 * entries that would land beyond max_blocks are skipped. */
spkv_status spkv_block_table_append(int32_t *tables, int32_t max_blocks, int32_t *lens, int32_t num_rows,
                                    const int32_t *rows, const int32_t *slots, int32_t n, int32_t page_size,
                                    void *stream);

/* ======================================================================
 * Decode attention.
 * ==================================================================== */

/* One decode step's batch.  Requests that share a prefix form a group whose
 * prefix sits in one HOT slab ([GKV] Section 3.4: each prefix records a HOT
 * base or a COLD marker).  A request with group -1 keeps its whole context
 * (prefix included) in the COLD pool ([GKV] Appendix B.10 fallback).
 * Membership is group_of alone: the library forms each group's member list
 * (ascending request id) itself, on the host for the plan and on the device
 * for the prefix contraction, so no separate member list can disagree with it.
 * The host copies must hold the same values as the device arrays. */
typedef struct spkv_batch {
    int32_t batch;                 /* B >= 0 */
    int32_t num_q_heads;           /* Hq, a multiple of Hkv, Hq/Hkv <= 8 */
    int32_t num_kv_heads;          /* Hkv, 1..16 */
    int32_t head_dim;              /* d: 64 or 128 */
    int32_t dtype;                 /* SPKV_DTYPE_* of q and of every K/V pool */
    float   scale;                 /* softmax scale applied to q.k, > 0 (usually 1/sqrt(d)) */
    const void *q;                 /* device [B, Hq, d] */

    int32_t num_groups;            /* ng, 0..512 */
    const int32_t *group_of;       /* device [B]: group of request b in [0, ng), or -1 */
    const int64_t *hot_base;       /* device [ng]: slab base (token slot) */
    const int32_t *hot_len;        /* device [ng]: prefix length Lp_g >= 0; one head's slab
                                      (Lp_g * d * element size) must stay below 4 GiB */
    const int32_t *host_group_of;  /* host copies of group_of, hot_base and hot_len */
    const int64_t *host_hot_base;
    const int32_t *host_hot_len;

    int32_t page_size;             /* COLD page size P >= 1 */
    int32_t max_blocks;            /* columns of block_tables */
    const int32_t *block_tables;   /* device [B, max_blocks], -1 padded */
    const int32_t *cold_lens;      /* device [B]: COLD tokens per request (the step's token included) */
    const int32_t *host_cold_lens; /* host copy of cold_lens */
} spkv_batch;

/* The pools attention reads (device memory, caller-owned), and the layer
 * this call attends: both pools hold num_layers layers in the layouts above,
 * with one HOT allocation and one COLD allocation for all of them. */
typedef struct spkv_kv {
    const void *k_hot;
    const void *v_hot;
    int64_t hot_capacity;          /* tokens */
    const void *k_cold;
    const void *v_cold;
    int64_t cold_slots;            /* num_pages * page_size (per layer) */
    int32_t num_layers;            /* L >= 1 */
    int32_t layer;                 /* 0 <= layer < L */
} spkv_kv;

/* Workspace bytes the decode calls below need for this batch in any mode
 * (partial attention states of the split plan).  0 on invalid input. */
size_t spkv_workspace_size(const spkv_batch *batch);

/* Cascade attention ([GKV] Section 2.3): per group, every member's queries
 * attend to the HOT slab once in one batched Q.K^T / P.V contraction
 * (bf16 MFMA); per request, the COLD suffix is attended by a paged pass; the
 * two partial states are merged by log-sum-exp ([GKV] Eq. (1)).  Requests
 * without a group take the paged pass over their COLD tokens only.
 * For float32 pools the prefix part is the same batched contraction (every
 * member's query rows against the slab, read once per group) in float32 on
 * the vector units; the per-group dispatcher only picks it when forced (its
 * cost constants are fitted to the bf16 kernels).  `lse` may be NULL. */
spkv_status spkv_cascade_decode(const spkv_batch *batch, const spkv_kv *kv, float *out, float *lse,
                                void *ws, size_t ws_bytes, void *stream);

/* Flat paged decode ([PKV] How it works, step 3; [GKV] Section 4.3 "SGLang
 * default"): each request attends its HOT prefix and then its COLD suffix in
 * one online-softmax pass, re-reading the shared prefix per request.  Output
 * equals spkv_cascade_decode up to rounding. */
spkv_status spkv_dense_decode(const spkv_batch *batch, const spkv_kv *kv, float *out, float *lse,
                              void *ws, size_t ws_bytes, void *stream);

/* Two-way log-sum-exp merge of partial states ([GKV] Eq. (1)): rows of
 * (o_a, lse_a) and (o_b, lse_b) -> (o, lse).  o_* are [rows, head_dim]
 * float32 and normalised; lse_* are natural-log float32 [rows], -inf for an
 * empty part.  Device pointers; outputs may alias inputs of the same row. */
spkv_status spkv_merge_states(const float *o_a, const float *lse_a, const float *o_b, const float *lse_b,
                              float *o, float *lse, int64_t rows, int32_t head_dim, void *stream);

/* ======================================================================
 * Per-step dispatch ([GKV] Section 3.6).  The paper computes
 * M_eff = B_step * n_q/kv (its Eq. (2)) every step and compares it with a
 * hardware-fitted constant.  Here the choice is cascade vs flat per prefix
 * group, from a cost model whose constants are data (re-fitted per GPU).
 * ==================================================================== */
#define SPKV_MODE_PER_GROUP      0   /* choose per group from the cost model */
#define SPKV_MODE_BATCH_GLOBAL   1   /* cascade only if the whole batch shares one prefix, else flat */
#define SPKV_MODE_FORCE_CASCADE  2
#define SPKV_MODE_FORCE_DENSE    3

typedef struct spkv_dispatch_params {
    int32_t mode;                  /* SPKV_MODE_* */
    int32_t min_group_requests;    /* cascade needs at least this many requests in the group */
    double  fixed_cost_us;         /* extra cost of the cascade path per step (launch + merge) */
    double  flat_gbps;             /* effective bandwidth of the flat pass over the prefix */
    double  prefix_gbps;           /* effective bandwidth of the prefix contraction */
    double  prefix_tflops;         /* effective bf16 MFMA rate of the prefix contraction */
    double  row_cost_ns;           /* cascade cost per query row of a group that takes it
                                      (its prefix partial states: written, then merged) */
    int32_t single_launch;         /* 1 (default): the paged pass and the prefix contraction run as one
                                      launch where the plan allows it (spkv_plan_info.single_launch),
                                      side by side in every launch block where the plan marks it
                                      co-resident (spkv_plan_info.co_resident), else the prefix blocks
                                      after the paged ranges; 2: one launch, never co-resident;
                                      0: always two launches. */
} spkv_dispatch_params;

/* Defaults fitted on MI355X (see the design notes for the fit). */
void spkv_dispatch_params_default(spkv_dispatch_params *p);

/* Host-only and pure: cascade_out[g] = 1 (cascade) or 0 (flat) for each group. */
spkv_status spkv_dispatch(const spkv_batch *batch, const spkv_dispatch_params *params, int32_t *cascade_out);

/* Dispatch, then run: groups chosen for cascade take the prefix contraction,
 * the others are folded into the flat pass; one merge finishes every row.
 * Where the plan allows it and params->single_launch is set, the paged pass
 * and the prefix contraction run as one launch.  Co-resident (the default
 * where the plan marks it): every launch block runs a paged block on four
 * waves and a prefix item on two or four more, the prefix in one key half,
 * so its values differ from the two launches' by rounding order only (within
 * the same bound of the exact result).  Otherwise the prefix blocks follow
 * the paged ranges in the grid and the results are bit-identical to two
 * launches.  spkv_cascade_decode uses the single launch wherever the plan
 * allows it.
 * cascade_out (host [ng], nullable) reports the choice. */
spkv_status spkv_decode_step(const spkv_batch *batch, const spkv_kv *kv, const spkv_dispatch_params *params,
                             float *out, float *lse, void *ws, size_t ws_bytes, void *stream,
                             int32_t *cascade_out);

/* The step's appends fused into the decode step ([PKV] How it works, steps
 * 1-3, then the step as above): the same results, pools, block tables and
 * lengths as spkv_append_tokens(k_new, v_new, host_slots, rows 0..B-1, ...,
 * block_tables, cold_lens) followed by spkv_decode_step, with one launch
 * fewer.  The paged pass reads request b's new token from row b of k_new /
 * v_new ([B, Hkv, d], device); the merge then writes it to COLD slot
 * host_slots[b] (host [B], the allocator's output) and advances the device
 * block table and length.  batch->host_cold_lens must already count the new
 * token; the device cold_lens and block tables must not.  bf16 only.
 * Returns SPKV_E_INVAL, before any launch, for a slot outside
 * [0, cold_slots), a length whose new token has no block-table column, a
 * COLD pool with Hkv * cold_slots >= 2^30, or float32 data.  Run
 * spkv_copy_blocks for the step's copy-on-write pairs first. */
spkv_status spkv_decode_step_append(const spkv_batch *batch, const spkv_kv *kv,
                                    const spkv_dispatch_params *params, const void *k_new, const void *v_new,
                                    const int32_t *host_slots, float *out, float *lse, void *ws,
                                    size_t ws_bytes, void *stream, int32_t *cascade_out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as spkv_decode_step_append, with the same results, but without a
 * workspace argument.  The partial states live in a static device array of
 * SPKV_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends (its address is looked up once per device with
 * hipGetSymbolAddress).  The call allocates nothing.  Returns SPKV_E_INVAL,
 * before any launch, when the step's plan needs more scratch than that
 * (spkv_plan_query reports workspace_bytes).  Every call on one device uses
 * the same array: calls that overlap on one device (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in the array
 * has to start at zero. */
#define SPKV_NOALLOC_SCRATCH_BYTES (32u << 20)
spkv_status spkv_decode_step_append_noalloc(const spkv_batch *batch, const spkv_kv *kv,
                                            const spkv_dispatch_params *params, const void *k_new,
                                            const void *v_new, const int32_t *host_slots, float *out, float *lse,
                                            void *stream, int32_t *cascade_out);

/* ======================================================================
 * The decode step as a HIP graph ([GKV] Appendix B.2b: per-backend graph
 * buffers in the serving engine).  The step's kernel arguments change every
 * step (lengths grow, slots move), so the graph is not replayed as recorded:
 * each call records the step on a private stream (recording enqueues no GPU
 * work), updates the instantiated graph's kernel nodes with this step's
 * arguments in place (hipGraphExecUpdate) when the step has the same launches
 * as the graph, re-instantiates it otherwise, and launches the graph on
 * `stream`.  The graph uses no memset nodes.
 * ==================================================================== */
typedef struct spkv_graph spkv_graph;

spkv_status spkv_graph_create(spkv_graph **out);
void        spkv_graph_destroy(spkv_graph *graph);
/* The same arguments, results and errors as spkv_decode_step_append, run as
 * the handle's graph; *instantiated_out (nullable) is 1 when the graph had to
 * be (re)instantiated instead of updated.  A handle is single-owner and not
 * thread-safe; the workspace must stay valid until the launch has run. */
spkv_status spkv_graph_decode_step_append(spkv_graph *graph, const spkv_batch *batch, const spkv_kv *kv,
                                          const spkv_dispatch_params *params, const void *k_new,
                                          const void *v_new, const int32_t *host_slots, float *out, float *lse,
                                          void *ws, size_t ws_bytes, void *stream, int32_t *cascade_out,
                                          int32_t *instantiated_out);

/* ======================================================================
 * Plan inspection and kernel timing (measurement support).
 * ==================================================================== */
typedef struct spkv_plan_info {
    int32_t flat_chunk;            /* virtual tokens per range of the paged pass (stream-K; largest
                                      sub-batch; flat_head_tokens count before each non-empty request) */
    int32_t flat_splits;           /* max paged-pass partials of one request (<= flat_split_cap) */
    int32_t prefix_chunk;          /* base keys per prefix work item (bf16 MFMA pass) */
    int32_t prefix_splits;         /* max prefix partials per row */
    int32_t prefix_waves;          /* waves per prefix work item (32 query rows each) */
    int32_t prefix_mtiles;         /* max row tiles per (group, KV head) */
    int64_t flat_items;            /* paged-pass work items (ranges x KV-head groups) */
    int64_t prefix_items;          /* non-empty prefix work items */
    int64_t workspace_bytes;       /* bytes this plan uses */
    int32_t flat_split_cap;        /* bound on the paged-pass partials of one request */
    int32_t flat_head_tokens;      /* start cost of one (range, request) piece in tokens: ranges are cut
                                      with this many virtual tokens before each non-empty request */
    int32_t prefix_split_cap;      /* per group: chunk = roundup(max(prefix_chunk, ceil(Lp / cap)), granule) */
    int32_t prefix_granule;
    int32_t prefix_key_halves;     /* 2: each prefix work item's key chunk is split over two wave sets whose
                                      states merge in LDS (one partial per row per item either way) */
    int32_t single_launch;         /* 1: the paged pass's ranges and the prefix blocks can run as one launch
                                      (bf16, head_dim 128, Hkv of 1, 2 or >= 4, one paged sub-batch of
                                      <= 256 requests, prefix tiles of 2 or 4 row waves with two key halves
                                      (groups of more than 32 query rows per KV head)); the
                                      paged ranges come first in the grid and the prefix blocks take CUs as
                                      ranges finish */
    int32_t co_resident;           /* 1: that one launch can run both roles in every launch block (four
                                      paged waves beside the prefix item's waves): the prefix items of
                                      cascade groups with a prefix, counted at prefix_mtiles for every
                                      group, number no more than the paged blocks */
    int32_t co_prefix_stages;      /* ring depth of the co-resident launch's prefix waves (tiles of 32
                                      keys): 3 beside paged rings of 3 stages, or 5 beside paged rings of 2
                                      when its prefix items (tiles of 4 row waves) hold more key tiles than
                                      a paged wave's range holds ring stages of 16 tokens; 0 when not
                                      co-resident */
} spkv_plan_info;

spkv_status spkv_plan_query(const spkv_batch *batch, const int32_t *cascade, spkv_plan_info *out);

/* Partial states the plan writes per request (host arrays of length B, filled
 * by the call): flat_parts[b] by the paged pass, prefix_parts[b] per query row
 * by the prefix part (0 without a cascade prefix).  The merge of request b
 * combines flat_parts[b] + prefix_parts[b] states per query row ([GKV] Eq. (1)
 * applied across all of them).  Either pointer may be NULL. */
spkv_status spkv_plan_parts(const spkv_batch *batch, const int32_t *cascade, int32_t *flat_parts,
                            int32_t *prefix_parts);

#define SPKV_KERNEL_PREFIX        0   /* prefix contraction (bf16 MFMA, or float32) */
#define SPKV_KERNEL_FLAT          1   /* paged pass: suffix part, or whole context when flat */
#define SPKV_KERNEL_MERGE         2   /* log-sum-exp merge of partial states */
#define SPKV_KERNEL_CACHE         3   /* hot_write / reshape_and_cache / copy_blocks / append_tokens */
#define SPKV_KERNEL_PAGED_PREFIX  4   /* paged pass and prefix contraction in one launch */
#define SPKV_NUM_KERNELS          5

/* When on, every launch is bracketed by HIP events on its stream. */
spkv_status spkv_timing_enable(int32_t on);
/* Waits for the recorded events and returns the summed duration (ms) and the
 * launch count of one kernel class since the last reset. */
spkv_status spkv_timing_read(int32_t kernel, double *total_ms, int64_t *launches);
spkv_status spkv_timing_reset(void);

/* Number of compute units of the current device (SPKV_E_HIP without a GPU). */
spkv_status spkv_device_cus(int32_t *cus_out);

/* Measured ceilings, for rooflines against what this device achieves beside
 * its published peaks.  Each is one launch on `stream`; time it with events
 * around the call.
 * spkv_probe_read: streams `bytes` bytes of device memory at `src` (16-byte
 * aligned, bytes a multiple of 16 and > 0) through nontemporal 16-byte
 * vector loads, each block of 4 waves taking contiguous 32 KB chunks in turn;
 * min(16 * CUs, chunks, sink_words / 4) blocks.  Wave w writes the XOR of
 * the 32-bit words it read to sink[w] (device uint32, sink_words >= 4
 * entries; entries past the launched waves are left as they are, so the XOR
 * of a zeroed sink is the checksum of the buffer).
 * spkv_probe_mfma: `waves` waves (a multiple of 4, > 0) each run `iters`
 * rounds of 8 independent v_mfma_f32_32x32x16_bf16 (8 x 32768 FLOPs per
 * round) from register operands and write one accumulator sum per wave to
 * sink[wave] (device float).  SPKV_E_INVAL on bad sizes. */
spkv_status spkv_probe_read(const void *src, size_t bytes, uint32_t *sink, int32_t sink_words, void *stream);
spkv_status spkv_probe_mfma(int32_t waves, int32_t iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SPKV_H */
