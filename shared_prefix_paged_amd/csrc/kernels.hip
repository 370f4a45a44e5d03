// HIP kernels for gfx950 (MI355X) and the device-op entry points of the C ABI.
//
// Decode attention over HOT/COLD storage (GraniKV paper, Sections 2.3, 3.2,
// 3.3, 3.5): the prefix part is one batched contraction of every member query
// of a prefix group against its contiguous HOT slab (bf16 MFMA, K/V tiles
// staged through LDS); the suffix part is a per-request paged pass over the
// COLD pool ("Paged KV cache" page, How it works step 3); partial states are
// combined with the log-sum-exp merge of the paper's Eq. (1).  The flat
// fallback runs the paged pass over [HOT prefix ; COLD suffix] per request.
//
// Internal conventions: scores are kept in log2 units (q.k * scale * log2 e)
// so exp2 maps to the hardware's v_exp_f32; partial LSE values stored in the
// workspace are base 2, and only outputs are converted to natural log.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "internal.h"

using spkv::fail;
using spkv::FlatLaunch;
using spkv::GroupMask;
using spkv::Plan;
using spkv::flat_parts;
using spkv::range_of;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFlatWavesMax = 4; // KV heads per flat block

struct Args {
    const void *q;
    int32_t B, Hq, Hkv, G;
    float scale_log2;
    int32_t ng;
    const int32_t *group_of;
    const int64_t *hot_base;
    const int32_t *hot_len;
    int32_t page_size, max_blocks;
    const int32_t *tables;
    const int32_t *cold_lens;
    const void *k_hot;
    const void *v_hot;
    int64_t hot_capacity;
    const void *k_cold;
    const void *v_cold;
    int64_t cold_slots;
    float *o_part;          // [B*Hq, splits_total, D]
    float *lse_part;        // [B*Hq, splits_total], base-2
    int32_t splits_total;
    int32_t prefix_splits;  // offset of the flat partials inside a row
    int32_t flat_splits;    // flat partial slots per row
    int32_t flat_tau, prefix_tau, prefix_granule;
    int32_t prefix_mode;    // 0: no prefix partials; 1: the prefix contraction's split rule
    GroupMask cascade;
    // Append mode (the step's new tokens not yet in the pools): every request
    // has one COLD token more than cold_lens counts, the last one, whose K/V
    // rows are row b of k_new / v_new [B, Hkv, d].
    const void *k_new;
    const void *v_new;
    int32_t append;
    // Layer of this call in pools of num_layers layers: the HOT slab of a
    // prefix at token slot base holds layer l's head h at row
    // base*Hkv*L + l*Lp*Hkv + h*Lp ([GKV] Section 3.2); k_cold / v_cold already
    // point at this layer's COLD pool.
    int32_t num_layers, layer;
    // Set when no request's paged-pass tokens include HOT slab rows: every
    // K/V row the bf16 paged pass reads is then a private COLD row, read once
    // per step, and is loaded with the non-temporal hint.
    int32_t cold_nt;
};

__device__ __forceinline__ bool mask_get(const GroupMask &m, int g) { return (m.bits[g >> 5] >> (g & 31)) & 1u; }

// First row of head h of this call's layer in a HOT slab at token slot base
// holding a prefix of lp tokens (rows of the pool's K or V buffer).
__device__ __forceinline__ int64_t slab_row(const Args &a, int64_t base, int lp, int h) {
    return base * a.Hkv * a.num_layers + (int64_t)a.layer * lp * a.Hkv + (int64_t)h * lp;
}

// Geometry of one request, clamped so that no index can leave its buffer.
struct Req {
    int g;          // group or -1
    int64_t base;   // HOT slab base
    int lp;         // HOT prefix length (0 without a group)
    int ls;         // COLD tokens
    bool casc;      // group takes the prefix contraction
};

// Load through the constant address space: the kernels never write these
// arrays, and a wave-uniform address then becomes a scalar load (counted by
// lgkmcnt, so it never waits for vector-memory DMAs in flight).
template <class T>
__device__ __forceinline__ T ld_const(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

__device__ __forceinline__ Req req_geo(const Args &a, int b) {
    Req r;
    int g = ld_const(a.group_of + b);
    r.g = (g >= 0 && g < a.ng) ? g : -1;
    r.base = 0;
    r.lp = 0;
    r.casc = false;
    if (r.g >= 0) {
        int64_t base = ld_const(a.hot_base + r.g);
        int lp = ld_const(a.hot_len + r.g);
        if (base >= 0 && lp > 0 && base + lp <= a.hot_capacity) {
            r.base = base;
            r.lp = lp;
        }
        r.casc = mask_get(a.cascade, r.g);
    }
    int ls = ld_const(a.cold_lens + b) + a.append;
    const int64_t cap = (int64_t)a.max_blocks * a.page_size;
    r.ls = ls < 0 ? 0 : (ls > cap ? (int)cap : ls);
    if (a.cold_slots < a.page_size) r.ls = 0;   // no COLD page to read
    return r;
}

// Tokens of request b the paged pass attends: [lo, hi) of [HOT prefix ; COLD
// suffix] - the COLD suffix, plus the HOT prefix when the request's group
// takes the flat pass instead of the prefix contraction.
__device__ __forceinline__ void flat_range(const Req &r, int &lo, int &hi) {
    lo = (r.g >= 0 && r.casc) ? r.lp : 0;
    hi = r.lp + r.ls;
}

template <int N>
__device__ __forceinline__ float dpp_sum(float v);

// Sum over aligned groups of N lanes (N = 8, 16, 32); every lane gets its group's sum.
template <>
__device__ __forceinline__ float dpp_sum<8>(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)); // row_half_mirror
    return v;
}
template <>
__device__ __forceinline__ float dpp_sum<16>(float v) {
    v = dpp_sum<8>(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)); // row_mirror
    return v;
}
template <>
__device__ __forceinline__ float dpp_sum<32>(float v) {
    v = dpp_sum<16>(v);
    v += __shfl_xor(v, 16, 64);
    return v;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// max(v[l], v[l ^ 32]) in every lane l (v_permlane32_swap exchanges the
// upper half of one register with the lower half of another).
__device__ __forceinline__ float max_of_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// Global->LDS DMA (global_load_lds_*): lane l's bytes land at M0 + size * l.
// The compiler does not track these loads, so every wait on them is an
// explicit s_waitcnt; loads the compiler does track are only ever counted
// conservatively by it (extra loads in flight make its waits stricter).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_char_t *)p;
}

// One wave-wide global->LDS copy: this lane's 16 bytes (at gbase + voff) land
// at lds_base + 16 * lane.  gbase and lds_base must be wave-uniform.  M0 (the
// LDS base of the copy) is saved and restored around the instruction; the
// s_nop covers the M0-write hazard.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Same with a 64-bit address per lane (any pool size).
__device__ __forceinline__ void dma16_at(const void *addr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(addr), "s"(lds_base)
        : "memory");
}

// 4 bytes per lane: lane l's dword (at gbase + voff) lands at lds_base + 4 * l.
// The same with the non-temporal hint, for rows that are read once per step.
__device__ __forceinline__ void dma16_at_nt(const void *addr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(addr), "s"(lds_base)
        : "memory");
}

__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory");
}

// Wait until at most N vector-memory loads of this wave are in flight and
// every LDS access it issued has completed.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Flat paged pass.  A block takes one token range of a stream-K split (see
// FlatLaunch) for up to 4 KV heads, one wave per head.  LPT lanes hold one
// token's K (or V) row as 16-byte pieces, so one wave-wide access covers TPW
// tokens; each group of LPT lanes keeps its own online-softmax state, and the
// groups are combined once per range.
//
// Memory pipeline: K/V rows are gathered straight into LDS by DMA (one 64-bit
// address per lane), through a ring of kFlatStages stages per wave that runs
// kFlatStages-1 stages ahead of the compute, so data in flight occupies no
// VGPRs.  A stage is one wave-wide DMA of K and one of V (TPW tokens, 2 KB).
// Row codes (HOT slab row or COLD slot row, bit 31 = HOT) are built per
// 64-token block, one token per lane; the block-table entries of the next
// block are DMA'd into LDS a block ahead, so nothing in the loop waits on a
// load the compiler tracks and all waits are explicit vmcnt counts.
// ---------------------------------------------------------------------------
constexpr int kFlatStages = 4;

template <bool BF16, int D>
struct FlatGeom {
    static constexpr int ESZ = BF16 ? 2 : 4;
    static constexpr int VEC = 16 / ESZ;         // elements per 16-byte piece
    static constexpr int LPT = D / VEC;          // lanes per token row
    static constexpr int TPW = 64 / LPT;         // tokens per stage
    static constexpr int SPB = 64 / TPW;         // stages per 64-token block
    static constexpr int ROWB = D * ESZ;         // bytes per K/V row
    static constexpr int STAGEB = 2048;          // K (1 KB) then V (1 KB)
    static constexpr int TABB = 256;             // 64 block-table entries
    static constexpr int WAVEB = kFlatStages * STAGEB + TABB;
    static_assert(TPW * ROWB == 1024, "a stage operand is one 1 KB wave-wide DMA");
    static_assert(kFlatStages - 1 < SPB, "prologue stays inside the first 64-token block");
    static_assert((kFlatStages & (kFlatStages - 1)) == 0, "ring index is a mask");
};

// Online softmax of the G query rows of KV head h over tokens [t0, t1) of
// request b; the normalised partial state goes to partial slot `slot`.
// `ring` is this wave's LDS area (FlatGeom::WAVEB bytes), `ring_off` its LDS
// address.
template <bool BF16, int D, int G>
__device__ __forceinline__ void attend_range(const Args &a, const Req &r, int b, int h, int t0, int t1, int slot,
                                             int lane, char *ring, uint32_t ring_off) {
    using FG = FlatGeom<BF16, D>;
    constexpr int S = kFlatStages;
    constexpr int VEC = FG::VEC, LPT = FG::LPT, TPW = FG::TPW, SPB = FG::SPB;
    constexpr float kRescaleSlack = 8.f;     // see the prefix kernel: exact for any reference

    const int sub = lane % LPT;              // 16-byte piece of the row
    const int grp = lane / LPT;              // token group inside the wave
    const int row0 = b * a.Hq + h * G;       // first query row of this head

    const char *khot = (const char *)a.k_hot;
    const char *vhot = (const char *)a.v_hot;
    const char *kcold = (const char *)a.k_cold;
    const char *vcold = (const char *)a.v_cold;
    const int32_t *table = a.tables + (int64_t)b * a.max_blocks;
    const int64_t num_pages = a.cold_slots / a.page_size;
    const uint32_t hot_row0 = (uint32_t)slab_row(a, r.base, r.lp, h);
    const int32_t *tab_lds = (const int32_t *)(ring + S * FG::STAGEB);
    const uint32_t tab_off = ring_off + S * FG::STAGEB;

    // Token of 64-block n taken by this lane (clamped into the range), and the
    // first block-table index the block needs.
    auto lane_token = [&](int n) { return min(t0 + 64 * n + lane, t1 - 1); };
    auto first_entry = [&](int n) { return (max(t0 + 64 * n, r.lp) - r.lp) / a.page_size; };
    auto block_has_cold = [&](int n) { return t0 + 64 * n < t1 && t0 + 64 * n + 63 >= r.lp; };
    auto code_of = [&](int t, int32_t entry) -> uint32_t {
        if (t < r.lp) return 0x80000000u | (hot_row0 + (uint32_t)t);
        int64_t page = entry;
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        return (uint32_t)((page * a.page_size + (t - r.lp) % a.page_size) * a.Hkv + h);
    };
    // Table entries e0 .. e0+63 of block n into the LDS table area.
    auto table_dma = [&](int n) {
        const int e = max(0, min(first_entry(n) + lane, a.max_blocks - 1));
        dma4(table, (uint32_t)e * 4u, tab_off);
    };
    // Row codes of block n from the LDS table (its DMA has landed).
    auto code_from_lds = [&](int n) -> uint32_t {
        const int t = lane_token(n);
        int32_t entry = 0;
        if (t >= r.lp) entry = tab_lds[max(0, min((t - r.lp) / a.page_size - first_entry(n), 63))];
        return code_of(t, entry);
    };

    // Query rows in registers, and the row codes of block 0, loaded (and
    // consumed) before any DMA is in flight.
    uint32_t qw[G][4];
    {
        const char *qb = (const char *)a.q + ((int64_t)row0 * D + sub * VEC) * FG::ESZ;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            u32x4_t v = *(const u32x4_t *)(qb + (int64_t)g * D * FG::ESZ);
            qw[g][0] = v.x; qw[g][1] = v.y; qw[g][2] = v.z; qw[g][3] = v.w;
        }
    }
    uint32_t code;
    {
        const int t = lane_token(0);
        int32_t entry = 0;
        if (t >= r.lp) entry = table[max(0, min((t - r.lp) / a.page_size, a.max_blocks - 1))];
        code = code_of(t, entry);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) asm volatile("" ::"v"(qw[g][0]), "v"(qw[g][1]), "v"(qw[g][2]), "v"(qw[g][3]));
    asm volatile("" ::"v"(code));

    // Stage j: tokens t0 + j*TPW + grp, LDS slot j % S.
    auto issue = [&](int j) {
        const int ti = (j % SPB) * TPW + grp;    // token inside its 64-block; lane ti holds its code
        const uint32_t c = (uint32_t)__shfl((int)code, ti, 64);
        const bool hot = c >> 31;
        const int64_t off = (int64_t)(c & 0x7fffffffu) * FG::ROWB + sub * 16;
        const uint32_t dst = ring_off + (uint32_t)((j & (S - 1)) * FG::STAGEB);
        dma16_at((hot ? khot : kcold) + off, dst);
        dma16_at((hot ? vhot : vcold) + off, dst + 1024);
    };

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
    }
    const float c2 = a.scale_log2;

    auto compute = [&](int j) {
        const char *st = ring + (j & (S - 1)) * FG::STAGEB + lane * 16;
        const u32x4_t kk = *(const u32x4_t *)st;
        const u32x4_t vv = *(const u32x4_t *)(st + 1024);
        const bool valid = j * TPW + grp < t1 - t0;
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d;
            if constexpr (BF16) {
                d = fdot2(qw[g][0], kk.x, 0.f);
                d = fdot2(qw[g][1], kk.y, d);
                d = fdot2(qw[g][2], kk.z, d);
                d = fdot2(qw[g][3], kk.w, d);
            } else {
                d = __uint_as_float(qw[g][0]) * __uint_as_float(kk.x);
                d = fmaf(__uint_as_float(qw[g][1]), __uint_as_float(kk.y), d);
                d = fmaf(__uint_as_float(qw[g][2]), __uint_as_float(kk.z), d);
                d = fmaf(__uint_as_float(qw[g][3]), __uint_as_float(kk.w), d);
            }
            d = dpp_sum<LPT>(d);
            sc[g] = valid ? d * c2 : -INFINITY;   // log2 units
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (sc[g] > m[g] + kRescaleSlack) {     // rare after the first tokens
                const float alpha = __builtin_amdgcn_exp2f(m[g] - sc[g]);
                m[g] = sc[g];
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[g][e] *= alpha;
            }
            // m = -inf only while every token seen is masked (then p = 0, not NaN)
            const float nm = m[g] == -INFINITY ? 0.f : m[g];
            sc[g] = __builtin_amdgcn_exp2f(sc[g] - nm);   // now the weight p
            l[g] += sc[g];
        }
        // P.V with each value element widened once and used by all G rows.
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const uint32_t w = vv[BF16 ? e / 2 : e];
            const float v = BF16 ? ((e & 1) ? bf16hi(w) : bf16lo(w)) : __uint_as_float(w);
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g][e] = fmaf(sc[g], v, acc[g][e]);
        }
    };

    const int n_st = (t1 - t0 + TPW - 1) / TPW;
    if (block_has_cold(1)) table_dma(1);
    const int pro = min(S - 1, n_st);
    for (int j = 0; j < pro; ++j) issue(j);
    int j = 0;
    for (; j + S - 1 < n_st; ++j) {
        wait_vm_lds<2 * (S - 2)>();   // stage j has landed: only stages j+1 .. j+S-2 may be in flight
        const int jn = j + S - 1;
        if (jn % SPB == 0) {         // first stage of block n: its table entries landed with stage j
            const int n = jn / SPB;
            code = code_from_lds(n);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // table read done before it is overwritten
            if (block_has_cold(n + 1)) table_dma(n + 1);
        }
        issue(jn);
        compute(j);
    }
    wait_vm_lds<0>();
    for (; j < n_st; ++j) compute(j);

    // Combine the TPW token groups of the wave (lanes sub, sub+LPT, ...).
    // Every DMA has landed (waited above), so the ring may be reused.
    const int srow = slot;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = m[g];
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
        const float muse = M == -INFINITY ? 0.f : M;
        const float sc = __builtin_amdgcn_exp2f(m[g] - muse);
        float lt = l[g] * sc;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = acc[g][e] * sc;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) {
            lt += __shfl_xor(lt, off, 64);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] += __shfl_xor(o[e], off, 64);
        }
        if (grp == 0) {
            const int64_t prow = (int64_t)(row0 + g) * a.splits_total + srow;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float *dst = a.o_part + prow * D + sub * VEC;
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                float4 w = make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
                *(float4 *)(dst + e) = w;
            }
            if (sub == 0) a.lse_part[prow] = lt > 0.f ? M + __log2f(lt) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Flat paged pass, bf16: scores and the weighted sum on MFMA.  One wave per
// KV head as above; the head's G query rows are the N columns of 16x16 MFMA
// tiles (columns n >= G carry zero queries and are never stored).  Per ring
// stage of 16 tokens:
//   S^T[token, row] = K_stage . Q^T          D/32 x v_mfma_f32_16x16x32_bf16
//   online softmax along tokens, in the log2 domain
//   O^T[dim, row]  += V_stage^T . P^T         D/16 x 2 x v_mfma_f32_16x16x16_bf16
// 16x16 MFMA operand layouts (n = lane % 16, q = lane / 16):
//   16x16x32: A[m][k] in lane m + 16*(k/8), element k%8; B[k][n] likewise
//   16x16x16: A[m][k] in lane m + 16*(k/4), element k%4; B[k][n] likewise
//   D[m][n] in lane n + 16*(m/4), register m%4
// so the score tile gives lane (n, q) row n's scores of tokens 4q .. 4q+3,
// which is exactly its B operand of the P.V step.  P goes to the MFMA as two
// bf16 terms (hi + lo), so the weights carry ~16 significant bits.  V^T comes
// from LDS by transposing reads (ds_read_b64_tr_b16: within 16 lanes, lane i
// receives element e of the 8-byte chunk addressed by lane 4e + i/4,
// component i%4).
//
// K and V rows are gathered into a per-wave LDS ring by DMA as in the float32
// pass; a DMA lands 1 KB (RPI rows), lane l at +16*l.  The 16-byte chunks of
// a stage row are XOR-swizzled (K: by the row, V: by pairs) so that the K
// reads (16 rows, one chunk each) and the transposing V reads (16 rows,
// 32 bytes each) spread over all LDS banks.
// ---------------------------------------------------------------------------
template <int D, int S_ = spkv::kFlatMfmaStages>
struct FlatMfmaGeom {
    static constexpr int S = S_;
    static constexpr int TOK = spkv::kFlatMfmaTokens;   // tokens per stage
    static constexpr int ROWB = D * 2;                   // bytes per K/V row
    static constexpr int OPB = TOK * ROWB;               // bytes per stage operand
    static constexpr int STAGEB = 2 * OPB;               // K then V
    static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWB;              // rows per wave-wide DMA
    static constexpr int NDMA = TOK / RPI;               // DMAs per operand per stage
    static constexpr int RPP = 256 / ROWB;               // rows per 256-byte bank period
    static constexpr int SPB = 64 / TOK;                 // stages per 64-token block
    static constexpr int TABB = 256;
    static constexpr int WAVEB = S * STAGEB + TABB;
    static constexpr int KS = D / 32;                    // score MFMAs per stage
    static constexpr int NDB = D / 16;                   // 16-dim output blocks
    static_assert(TOK == 16, "one 16x16 score tile per stage");
    static_assert(S >= 2 && S - 1 < SPB, "prologue stays inside the first 64-token block");
};
static_assert(FlatMfmaGeom<128>::WAVEB == spkv::flat_mfma_wave_bytes(128), "plan and kernel agree on the ring");
static_assert(FlatMfmaGeom<64>::WAVEB == spkv::flat_mfma_wave_bytes(64), "plan and kernel agree on the ring");

// Physical chunk of logical chunk c in stage row r (an involution in c).
template <int D>
__device__ __forceinline__ int kswz(int r, int c) {
    using F = FlatMfmaGeom<D>;
    return c ^ ((r / F::RPP) & (F::CPR - 1));
}
template <int D>
__device__ __forceinline__ int vswz(int r, int c) {
    using F = FlatMfmaGeom<D>;
    return c ^ (2 * ((r / F::RPP) & (F::CPR / 2 - 1)));
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_of_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_of_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// APP (append mode): request b's new token, the last of its [HOT ; COLD]
// tokens, is not in the pools yet (the merge launch lands it).  The piece that
// ends with it loads the head's K/V rows of the token from k_new / v_new at
// its start and, once its last stage has landed, writes them over the token's
// row of that stage in LDS (the token's DMA lanes fetched a placeholder row).
template <int D, int G, bool APP, bool NT, int S_ = spkv::kFlatMfmaStages>
__device__ __forceinline__ void attend_range_mfma(const Args &a, const Req &r, int b, int h, int t0, int t1,
                                                  int slot, int lane, char *ring, uint32_t ring_off) {
    using F = FlatMfmaGeom<D, S_>;
    constexpr int S = F::S, TOK = F::TOK, SPB = F::SPB, NDMA = F::NDMA, KS = F::KS, NDB = F::NDB;
    constexpr float kRescaleSlack = 8.f;     // see the prefix kernel: exact for any reference
    static_assert(G >= 1 && G <= 16, "query rows of a head fit the 16 MFMA columns");

    const int n = lane & 15;                 // query row of the head (padding when >= G)
    const int q = lane >> 4;                 // 16-lane group
    const int row0 = b * a.Hq + h * G;

    const char *khot = (const char *)a.k_hot;
    const char *vhot = (const char *)a.v_hot;
    const char *kcold = (const char *)a.k_cold;
    const char *vcold = (const char *)a.v_cold;
    const int32_t *table = a.tables + (int64_t)b * a.max_blocks;
    const int64_t num_pages = a.cold_slots / a.page_size;
    const uint32_t hot_row0 = (uint32_t)slab_row(a, r.base, r.lp, h);
    const int32_t *tab_lds = (const int32_t *)(ring + S * F::STAGEB);
    const uint32_t tab_off = ring_off + S * F::STAGEB;

    // Row codes (HOT slab row, bit 31 set, or COLD slot row), one token of the
    // current 64-token block per lane, exactly as in the float32 pass.
    auto lane_token = [&](int nb) { return min(t0 + 64 * nb + lane, t1 - 1); };
    auto first_entry = [&](int nb) { return (max(t0 + 64 * nb, r.lp) - r.lp) / a.page_size; };
    auto block_has_cold = [&](int nb) { return t0 + 64 * nb < t1 && t0 + 64 * nb + 63 >= r.lp; };
    // Row codes: bit 31 HOT slab row, else a COLD slot row.
    auto code_of = [&](int t, int32_t entry) -> uint32_t {
        if (t < r.lp) return 0x80000000u | (hot_row0 + (uint32_t)t);
        if (APP && t == r.lp + r.ls - 1) return (uint32_t)h;   // placeholder: slot 0, replaced in LDS
        int64_t page = entry;
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        return (uint32_t)((page * a.page_size + (t - r.lp) % a.page_size) * a.Hkv + h);
    };
    auto table_dma = [&](int nb) {
        const int e = max(0, min(first_entry(nb) + lane, a.max_blocks - 1));
        dma4(table, (uint32_t)e * 4u, tab_off);
    };
    auto code_from_lds = [&](int nb) -> uint32_t {
        const int t = lane_token(nb);
        int32_t entry = 0;
        if (t >= r.lp) entry = tab_lds[max(0, min((t - r.lp) / a.page_size - first_entry(nb), 63))];
        return code_of(t, entry);
    };

    // Q^T as the B operand of the score MFMAs: lane (n, q) holds elements
    // 32s + 8q .. 32s + 8q + 7 of query row n for step s (zeros for n >= G).
    // Loaded, with the row codes of block 0, before any DMA is in flight.
    bf16x8_t qb[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + (int64_t)(row0 + min(n, G - 1)) * D + 8 * q;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4_t v = n < G ? *(const u32x4_t *)(qp + 32 * s) : u32x4_t{0, 0, 0, 0};
            qb[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
    uint32_t code;
    {
        const int t = lane_token(0);
        int32_t entry = 0;
        if (t >= r.lp) entry = table[max(0, min((t - r.lp) / a.page_size, a.max_blocks - 1))];
        code = code_of(t, entry);
    }
    // The new token's K/V rows of this head: lane c < CPR holds 16-byte chunk c.
    const bool lands = APP && t1 == r.lp + r.ls;   // this piece ends with the new token
    u32x4_t new_k = {0, 0, 0, 0}, new_v = {0, 0, 0, 0};
    if constexpr (APP) {
        if (lands && lane < F::CPR) {
            const int64_t src = ((int64_t)b * a.Hkv + h) * F::CPR + lane;
            new_k = ((const u32x4_t *)a.k_new)[src];
            new_v = ((const u32x4_t *)a.v_new)[src];
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qb[s])));
    asm volatile("" ::"v"(code));

    // Loop-invariant offsets.  DMA i of an operand lands stage rows
    // RPI*i .. RPI*i + RPI-1; this lane writes row RPI*i + lane / CPR at
    // physical chunk lane % CPR and so fetches the logical chunk kept there.
    uint32_t ksrc[NDMA], vsrc[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int rr = F::RPI * i + lane / F::CPR, p = lane % F::CPR;
        ksrc[i] = (uint32_t)(kswz<D>(rr, p) << 4);
        vsrc[i] = (uint32_t)(vswz<D>(rr, p) << 4);
    }
    // LDS reads (absolute LDS addresses of ring slot 0).  K for score step s:
    // row n (token), logical chunk 4s + q.  V for output block db: lane
    // (j = n, q) reads row 4q + j/4, bytes 32*db + 8*(j%4) of the row, i.e.
    // logical chunk 2*db + (j%4)/2 at byte 8*(j%2).
    uint32_t krd[KS], vrd[NDB];
#pragma unroll
    for (int s = 0; s < KS; ++s) krd[s] = ring_off + (uint32_t)(n * F::ROWB + (kswz<D>(n, 4 * s + q) << 4));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int rr = 4 * q + n / 4;
        vrd[db] = ring_off + (uint32_t)(F::OPB + rr * F::ROWB + (vswz<D>(rr, 2 * db + (n & 3) / 2) << 4) + 8 * (n & 1));
    }

    // Stage j: tokens t0 + 16j .. t0 + 16j + 15 into ring slot j % S.
    auto issue = [&](int j) {
        const uint32_t dst = ring_off + (uint32_t)(((unsigned)j % (unsigned)S) * F::STAGEB);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int ti = (j % SPB) * TOK + F::RPI * i + lane / F::CPR;   // token inside its 64-block
            const uint32_t c = (uint32_t)__shfl((int)code, ti, 64);
            const bool hot = c >> 31;
            const int64_t off = (int64_t)(c & 0x7fffffffu) * F::ROWB;
            if constexpr (NT) {   // the host found no HOT row in this launch; the pool select stays
                dma16_at_nt((hot ? khot : kcold) + off + ksrc[i], dst + 1024u * i);
                dma16_at_nt((hot ? vhot : vcold) + off + vsrc[i], dst + F::OPB + 1024u * i);
            } else {
                dma16_at((hot ? khot : kcold) + off + ksrc[i], dst + 1024u * i);
                dma16_at((hot ? vhot : vcold) + off + vsrc[i], dst + F::OPB + 1024u * i);
            }
        }
    };

    f32x4_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;
    const int nvalid = t1 - t0;
    typedef v4i16_t __attribute__((address_space(3))) *lds_v4i16_ptr;
    typedef bf16x8_t __attribute__((address_space(3))) *lds_bf16x8_ptr;

    // Stage j from ring slot st (st == j % S, a constant after unrolling).
    auto compute = [&](int j, int st) {
        // All LDS reads of the stage first (their latencies overlap), then the math.
        bf16x8_t kf[KS];
        s16x4_t va[NDB];
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[s] = *(lds_bf16x8_ptr)(uintptr_t)(krd[s] + st * F::STAGEB);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            va[db] = __builtin_bit_cast(s16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_v4i16_ptr)(uintptr_t)(vrd[db] + st * F::STAGEB)));
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qb[s], sacc, 0, 0, 0);
        float sv[4];
        const int tok = j * TOK + 4 * q;         // first of this lane's four tokens, relative to t0
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = tok + i < nvalid ? sacc[i] * c2 : -INFINITY;
        const float mx = max_of_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        const bool grow = mx > m_run + kRescaleSlack;
        if (__any(grow)) {
            const float mnew = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
            m_run = mnew;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
        l_run += (p[0] + p[1]) + (p[2] + p[3]);
        const bf16x2_t h01 = {(__bf16)p[0], (__bf16)p[1]}, h23 = {(__bf16)p[2], (__bf16)p[3]};
        const uint32_t w01 = __builtin_bit_cast(uint32_t, h01), w23 = __builtin_bit_cast(uint32_t, h23);
        const bf16x2_t l01 = {(__bf16)(p[0] - bf16lo(w01)), (__bf16)(p[1] - bf16hi(w01))};
        const bf16x2_t l23 = {(__bf16)(p[2] - bf16lo(w23)), (__bf16)(p[3] - bf16hi(w23))};
        const s16x4_t phi = __builtin_bit_cast(s16x4_t, u32x2_t{w01, w23});
        const s16x4_t plo = __builtin_bit_cast(
            s16x4_t, u32x2_t{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], phi, oacc[db], 0, 0, 0);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], plo, oacc[db], 0, 0, 0);
        }
    };

    const int n_st = (nvalid + TOK - 1) / TOK;
    if (block_has_cold(1)) table_dma(1);
    const int pro = min(S - 1, n_st);
    for (int j = 0; j < pro; ++j) issue(j);
    for (int j0 = 0; j0 < n_st; j0 += S) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const int j = j0 + st;
            if (j >= n_st) break;
            const int jn = j + S - 1;
            if (jn < n_st) {
                wait_vm_lds<2 * NDMA * (S - 2)>();   // stage j landed: only stages j+1 .. j+S-2 in flight
                if (jn % SPB == 0) {                 // first stage of block jn/SPB: its table entries landed
                    const int nb = jn / SPB;
                    code = code_from_lds(nb);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // table read before it is overwritten
                    if (block_has_cold(nb + 1)) table_dma(nb + 1);
                }
                issue(jn);
            } else {
                wait_vm_lds<0>();
            }
            if (APP && lands && j == n_st - 1 && lane < F::CPR) {
                // the last stage has landed (every DMA waited for): the new
                // token's row, at its swizzled chunk positions, over the placeholder
                typedef u32x4_t __attribute__((address_space(3))) *lds_u32x4_ptr;
                const int rn = (t1 - 1) - t0 - j * TOK;
                const uint32_t row = ring_off + (uint32_t)(st * F::STAGEB + rn * F::ROWB);
                *(lds_u32x4_ptr)(uintptr_t)(row + (kswz<D>(rn, lane) << 4)) = new_k;
                *(lds_u32x4_ptr)(uintptr_t)(row + F::OPB + (vswz<D>(rn, lane) << 4)) = new_v;
            }
            compute(j, st);
        }
    }

    // Every DMA has landed (the last stages waited for all), so the ring may
    // be reused.  The four lane groups hold disjoint dims of the same rows and
    // the same reference m_run; only the normaliser needs their sum.
    const float lt = sum_of_groups(l_run);
    if (n < G) {
        const int64_t prow = (int64_t)(row0 + n) * a.splits_total + slot;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        float *dst = a.o_part + prow * D + 4 * q;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *(float4 *)(dst + 16 * db) =
                make_float4(oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv);
        if (q == 0) a.lse_part[prow] = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
    }
}

// Per-request host data of one sub-batch's merge, in its kernel arguments
// (entry i is request b0 + i):
//  - slots: the step's new COLD slot (append mode), checked on the host (in
//    range, room in the block table);
//  - prefix_np: partial states of the MFMA prefix pass, from the host copies
//    of the group arrays, so no merging wave waits on a geometry load;
//  - flat_np: partial states of the paged pass (its ranges over the request,
//    from the launch's offsets), so no merging wave divides 64-bit integers.
struct MergeRows {
    int32_t slots[spkv::kFlatArgReqs];
    uint8_t prefix_np[spkv::kFlatArgReqs];
    uint8_t flat_np[spkv::kFlatArgReqs];
};

// Occupancy, float32: 4 waves per SIMD (<= 128 VGPRs) up to G = 6, 3 above;
// the LDS ring (4 x 8.25 KB per block of 4 waves) admits 4 blocks per CU.
// bf16: the LDS ring (4 x 8 KB per wave for d = 128) admits one or two
// blocks per CU, so registers are not the limit.
// One block of the paged pass: range k of the stream-K split, head group hy;
// wave `wave` (< kFlatWavesMax) of it takes KV head hy * kFlatWavesMax + wave
// with its ring at smem + wave * WAVEB.
template <bool BF16, int D, int G, bool APP, bool NT, int S_ = spkv::kFlatMfmaStages>
__device__ __forceinline__ void flat_block(const Args &a, const FlatLaunch &fl, const int k, const int hy,
                                           const int wave, const int lane, char *smem) {
    const int h = hy * kFlatWavesMax + wave;
    if (h >= a.Hkv) return;
    constexpr int WAVEB = BF16 ? FlatMfmaGeom<D, S_>::WAVEB : FlatGeom<BF16, D>::WAVEB;
    char *ring = smem + wave * WAVEB;
    const uint32_t ring_off = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(ring));
    const int64_t T = fl.total;
    const int nb = fl.blocks;
    const int64_t s0 = (T * k) / nb, s1 = (T * (k + 1)) / nb;
    if (s0 >= s1) return;
    // First request whose tokens reach past s0: the number of requests that
    // end at or before s0 (offs is non-decreasing), counted in one pass
    // instead of a chain of dependent loads.
    constexpr int NQW = (spkv::kFlatArgReqs + 63) / 64;
    int ends[NQW];
#pragma unroll
    for (int j = 0; j < NQW; ++j) ends[j] = fl.offs[min(lane + 64 * j, fl.nreq - 1) + 1];   // all loads in flight
    int i = 0;
#pragma unroll
    for (int j = 0; j < NQW; ++j) i += __popcll(__ballot(lane + 64 * j < fl.nreq && ends[j] <= s0));
    const int slot0 = a.prefix_splits;     // the paged pass's partial slots follow the prefix contraction's
    for (; i < fl.nreq; ++i) {
        const int64_t o0 = (int64_t)fl.offs[i] + fl.head, o1 = fl.offs[i + 1];
        if (o0 >= s1) break;
        const int64_t lo_s = s0 > o0 ? s0 : o0, hi_s = s1 < o1 ? s1 : o1;
        if (hi_s <= lo_s) continue;
        const int slot = k - range_of(o0, T, nb);
        if (slot < 0 || slot >= fl.max_parts) continue;   // cannot happen for a consistent plan
        const int b = fl.b0 + i;
        const Req r = req_geo(a, b);
        int lo, hi;
        flat_range(r, lo, hi);
        const int t0 = lo + (int)(lo_s - o0);
        const int t1 = min(hi, lo + (int)(hi_s - o0));   // device data shorter than the plan: clamp
        if (t1 <= t0) continue;
        if constexpr (BF16)
            attend_range_mfma<D, G, APP, NT, S_>(a, r, b, h, t0, t1, slot0 + slot, lane, ring, ring_off);
        else attend_range<BF16, D, G>(a, r, b, h, t0, t1, slot0 + slot, lane, ring, ring_off);
    }
}

template <bool BF16, int D, int G, bool APP = false, bool NT = false>
__global__ __launch_bounds__(256, (BF16 ? 2 : (G <= 6 ? 4 : 3))) void flat_kernel(Args a, FlatLaunch fl) {
    extern __shared__ __attribute__((aligned(1024))) char flat_smem[];
    flat_block<BF16, D, G, APP, NT>(a, fl, blockIdx.x, blockIdx.y, threadIdx.x >> 6, threadIdx.x & 63, flat_smem);
}

// ---------------------------------------------------------------------------
// Prefix contraction on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Block = W waves; wave w owns 32 query rows (rows of a prefix group are
// member-major: row = member * G + head-in-group).  Per 32-key tile:
//   S^T[key, row] = K_tile . Q^T   (A = K rows from LDS, B = Q in registers)
//   online softmax along keys: each lane holds one query row's 16 scores
//   O^T[d, row]  += V_tile^T . P^T (A = V from LDS by transposing reads,
//                                    B = P from the S^T accumulators in bf16)
// MFMA 32x32 operand layout: A[m][k] lives in lane m + 32*(k/8), element
// k%8; B[k][n] in lane n + 32*(k/8); D[m][n] in lane n + 32*((m/4)%2),
// register (m/8)*4 + m%4.  K rows are placed in LDS with bits 2 and 3 of the
// key index swapped, so accumulator register j of lane l holds key
// 16*(j/8) + 8*(l/32) + j%8, and registers 8*kb..8*kb+7 are already the P
// operand of the kb-th 16-key step.
//
// K/V tiles stream through a ring of LDS stages filled by global->LDS DMA
// (global_load_lds_dwordx4: lane l of a wave-wide load lands at base + 16*l),
// several tiles ahead of the MFMAs.  The 16-byte chunks of each LDS row are
// XOR-swizzled by row so that the K reads (16 B, 32 rows) and the transposing
// V reads (ds_read_b64_tr_b16: within 16 lanes, lane i receives element e of
// the 4x16-bit chunk addressed by lane 4e + i/4, component i%4) hit distinct
// banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swap_bits23(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// V tile chunk placement.  Logical 16-byte chunk c of LDS row r sits at
// physical chunk vchunk_phys(r, c); the transposing reads of one 16-lane group
// touch 4 consecutive rows x one 32-byte chunk pair, and the two groups read
// in the same cycle use pairs of opposite parity.  With 8 pairs per row
// (d = 128) the pair is rotated by 2 * (r % 4), so the 8 (row, pair)
// combinations of a cycle land on 8 distinct bank groups; with 4 pairs
// (d = 64) it is XOR-ed with r % 4.
template <int CPR>
__device__ __forceinline__ int vchunk_phys(int r, int c) {
    constexpr int NP = CPR / 2;
    const int m = c >> 1;
    const int pm = NP == 8 ? ((m + 2 * (r & 3)) & 7) : (m ^ (r & (NP - 1)));
    return 2 * pm + (c & 1);
}
template <int CPR>
__device__ __forceinline__ int vchunk_logical(int r, int p) {
    constexpr int NP = CPR / 2;
    const int pm = p >> 1;
    const int m = NP == 8 ? ((pm - 2 * (r & 3)) & 7) : (pm ^ (r & (NP - 1)));
    return 2 * m + (p & 1);
}

// SPLIT_P: P is rounded to bf16 for the P.V MFMA.  Its relative rounding error
// (2^-8) averages out over long prefixes; for short ones (few keys per row)
// P is carried as two bf16 terms, hi + lo, and P.V takes two MFMA passes.
// KH = 2: the block's key chunk is cut in two halves, each taken by W waves
// over the same W x 32 query rows with a ring of its own; the halves merge
// their states through LDS ([GKV] Eq. (1)) before one partial is written, so
// a row gets half as many partial states at the same number of waves per CU.
constexpr int kPrefixStages = 4;
constexpr int kMemberWin = 40;                 // >= 32 rows / G + 1 members
template <int D, int KH, int STAGES = kPrefixStages>
constexpr int prefix_ring_bytes() { return KH * STAGES * 2 * spkv::kPrefixKeyTile * D * 2; }

// Barrier of the W prefix waves of a block that also holds waves of another
// role (which never reach it): a counter in LDS that only grows.  The k-th
// barrier of each wave adds one and waits until the count reaches W * k.
// Every prefix wave passes the same number of barriers; the wait still gives
// up after a bounded number of polls, so no wave can wait forever.
__device__ __forceinline__ void waves_barrier(uint32_t *ctr, uint32_t target) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS reads of the tile before it arrives
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int poll = 0; poll < (1 << 22); ++poll) {
        const uint32_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// One block of the prefix contraction: key split s, row tile mt, (group, KV
// head) gz, run by waves wave_id = 0 .. W * KH - 1.  smem:
// prefix_ring_bytes<D, KH, STAGES>() bytes of LDS (1 KB aligned); member_win:
// W * KH windows of kMemberWin entries in LDS.  SWB: the block also runs
// waves of another role, so the prefix waves meet at waves_barrier on the
// LDS counter `bar` instead of the block-wide hardware barrier (one key half
// only).
template <int D, int W, bool SPLIT_P, int KH, int STAGES = kPrefixStages, bool SWB = false, bool PIPE = false>
__device__ __forceinline__ void prefix_block(const Args &a, const int s, const int mt, const int gz,
                                             const int wave_id, char *smem, int32_t (*member_win)[kMemberWin],
                                             uint32_t *bar = nullptr) {
    constexpr int NT = spkv::kPrefixKeyTile;   // 32 keys per tile
    constexpr int KS = D / 16;                 // MFMA k-steps for Q.K
    constexpr int NDB = D / 32;                // 32-column blocks of the output
    constexpr int ROWB = D * 2;                // bytes per K/V row
    constexpr int TILEB = NT * ROWB;           // bytes per K (or V) tile
    constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;              // rows per wave-wide DMA
    constexpr int IPW = NT / RPI / W;          // DMAs per wave per tile per operand
    static_assert(IPW >= 1 && (NT / RPI) % W == 0, "tile must split evenly over the waves");
    constexpr int AHEAD = (STAGES - 2) * 2 * IPW;   // DMAs issued after a tile's own
    static_assert(KH == 1 || KH == 2, "one or two key halves");
    static_assert(prefix_ring_bytes<D, KH, STAGES>() == KH * STAGES * 2 * TILEB, "ring size");
    static_assert(STAGES >= 3, "one tile in flight besides the one computed and the one issued");
    static_assert(!SWB || KH == 1, "the two-half exchange uses the hardware barrier");

    const int g = gz / a.Hkv;
    const int h = gz % a.Hkv;
    if (g >= a.ng || !mask_get(a.cascade, g)) return;
    const int64_t base = a.hot_base[g];
    const int lp = a.hot_len[g];
    if (lp <= 0 || base < 0 || base + lp > a.hot_capacity) return;
    const int chunk = spkv::chunk_for(lp, a.prefix_tau, spkv::kPrefixSplitCap, NT);
    const int nsplit = spkv::splits_for(lp, chunk);
    if (s >= nsplit) return;
    const int wave = wave_id % W;            // row wave (32 query rows)
    const int khalf = wave_id / W;           // key half
    const int lane = threadIdx.x & 63;
    uint32_t bar_k = 0;                      // barriers passed (SWB)
    // Tiles of the block's chunk: the first ceil(n/2) to half 0, the rest to
    // half 1.  Every wave runs nt_loop steps (a half with fewer tiles only
    // takes part in the barriers), so the barrier count is the same for all.
    const int kc0 = s * chunk;
    const int kc1 = min(lp, kc0 + chunk);
    const int nt_all = (kc1 - kc0 + NT - 1) / NT;
    const int nt_loop = KH == 1 ? nt_all : (nt_all + 1) / 2;
    const int k0 = kc0 + (khalf ? nt_loop * NT : 0);
    const int k1 = khalf ? kc1 : min(kc1, kc0 + nt_loop * NT);
    const int ntiles = khalf ? nt_all - nt_loop : nt_loop;
    const int half = lane >> 5;
    const int col = lane & 31;

    const char *kh = (const char *)a.k_hot + slab_row(a, base, lp, h) * ROWB;
    const char *vh = (const char *)a.v_hot + slab_row(a, base, lp, h) * ROWB;
    // kh / vh are wave-uniform (kernel arguments and block indices only), so
    // they live in SGPRs as the DMA's "s" operand requires.  (The readfirstlane
    // builtin is 32-bit and must not be applied to these 64-bit pointers.)
    const uint32_t smem0 =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(smem + khalf * STAGES * 2 * TILEB));

    // Per-lane source offsets and LDS placement of the DMAs, fixed for the
    // whole range (K row r of a tile holds key swap_bits23(r); the 16-byte
    // chunks of a row sit at their swizzled positions).  Per tile only the
    // wave-uniform source base moves.
    uint32_t ksrc[IPW], vsrc[IPW], wdst[IPW];
    int krow[IPW], vrow[IPW];
    {
        const int p = lane % CPR;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int r0 = (wave * IPW + i) * RPI;
            const int r = r0 + lane / CPR;
            krow[i] = swap_bits23(r);
            vrow[i] = r;
            ksrc[i] = (uint32_t)(krow[i] * ROWB + ((p ^ (r % CPR)) << 4));
            vsrc[i] = (uint32_t)(r * ROWB + (vchunk_logical<CPR>(r, p) << 4));
            wdst[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(r0 * ROWB));
        }
    }
    // Tile t of the range into LDS stage st.  In the last tile of a range that
    // ends inside it, rows past the end re-read the last valid key (in bounds;
    // those keys are masked before the softmax).
    auto issue = [&](int t, int st) {
        const int kt = k0 + t * NT;
        const char *kg = kh + (int64_t)kt * ROWB;
        const char *vg = vh + (int64_t)kt * ROWB;
        const uint32_t kst = smem0 + (uint32_t)(st * 2 * TILEB), vst = kst + TILEB;
        if (kt + NT <= k1) {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                dma16(kg, ksrc[i], kst + wdst[i]);
                dma16(vg, vsrc[i], vst + wdst[i]);
            }
        } else {
            const int last = k1 - 1 - kt;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int kr = min(krow[i], last), vr = min(vrow[i], last);
                dma16(kg, ksrc[i] + (uint32_t)((kr - krow[i]) * ROWB), kst + wdst[i]);
                dma16(vg, vsrc[i] + (uint32_t)((vr - vrow[i]) * ROWB), vst + wdst[i]);
            }
        }
    };

    // Prologue.  The compiler waits for its own loads with vmcnt(0), which
    // also covers every DMA in flight, so the group scan and Q (loads it
    // tracks) are read while only tile 0 is in flight, and tiles 1 .. STAGES-2
    // follow once Q has landed.
    if (ntiles > 0) issue(0, 0);

    // The group's members are the requests whose group_of is g, in ascending
    // id ([GKV] Section 3.4); query row r of the group belongs to member r / G.
    // One scan of group_of (64 requests per wave-wide load, several loads in
    // flight) counts the members and writes the ids this wave's 32 rows need,
    // member ranks [kw0, kw0 + kWin), to its LDS window.
    constexpr int kWin = kMemberWin;
    int32_t *win = member_win[wave_id];
    const int kw0 = (mt * 32 * W + wave * 32) / a.G;
    int count = 0;                             // wave-uniform
    for (int c0 = 0; c0 < a.B; c0 += 256) {
        int gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = c0 + 64 * u + lane;
            gv[u] = i < a.B ? a.group_of[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool mine = gv[u] == g;
            const uint64_t m = __ballot(mine);
            const int rank = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (mine && rank >= kw0 && rank < kw0 + kWin) win[rank - kw0] = c0 + 64 * u + lane;
            count += __popcll(m);
        }
    }
    const int M = count * a.G;
    if (mt * 32 * W >= M) {                    // block-uniform: every wave counted the same members
        wait_vmcnt<0>();                       // tile 0's DMA has landed before the LDS is released
        return;
    }
    __builtin_amdgcn_wave_barrier();           // the window's writes (other lanes) before its reads
    asm volatile("" ::: "memory");

    // This lane's query row (column of S^T / O^T).
    const int row = mt * 32 * W + wave * 32 + col;
    const bool row_ok = row < M;
    int qb = 0, qj = 0;
    if (row_ok) {
        const int mb = win[row / a.G - kw0];
        qb = max(0, min(mb, a.B - 1));
        qj = h * a.G + row % a.G;
    }
    bf16x8_t qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)qb * a.Hq + qj) * D + half * 8;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            u32x4_t v = row_ok ? *(const u32x4_t *)(qp + k * 16) : u32x4_t{0, 0, 0, 0};
            qf[k] = __builtin_bit_cast(bf16x8_t, v);
        }
        // Consume Q here so the compiler waits for its loads now, before the
        // next DMAs are issued, and not inside the loop.
#pragma unroll
        for (int k = 0; k < KS; ++k) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qf[k])));
    }
#pragma unroll
    for (int t = 1; t < STAGES - 1; ++t)
        if (t < ntiles) issue(t, t);

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    // Running reference max (log2 units) and normaliser.  The reference only
    // moves when a row's max grows by more than kRescaleSlack: any reference
    // gives the same O = sum 2^(s-m) v / sum 2^(s-m), and the slack bounds the
    // un-normalised terms by 2^kRescaleSlack.
    constexpr float kRescaleSlack = 8.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;

    // Loop-invariant LDS read offsets.  K: lane (col, half) reads 16 bytes of
    // key row col per k-step.  V (transposing reads): rows r1 and r1 + 4 of
    // the first 16-key step and r1 + 16, r1 + 20 of the second share one chunk
    // placement (it depends on the row modulo 4), so one offset per 32-column
    // block serves all four; the rest are immediates.
    uint32_t kofs[KS], vofs[NDB];
#pragma unroll
    for (int k = 0; k < KS; ++k) kofs[k] = (uint32_t)(col * ROWB + (((2 * k + half) ^ (col % CPR)) << 4));
    {
        const int g16 = lane >> 4, j16 = lane & 15;
        const int r1 = 8 * (g16 >> 1) + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int dpiece = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
            const int c = dpiece >> 3, inner = (dpiece & 7) * 2;
            vofs[db] = (uint32_t)(r1 * ROWB + (vchunk_phys<CPR>(r1, c) << 4) + inner);
        }
    }
    const lds_char_t *lsm = (const lds_char_t *)(smem + khalf * STAGES * 2 * TILEB);
    constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0) in bf16

    // One tile step, in parts: the K fragments of a tile from ring stage st;
    // its scores S^T = K . Q^T; the keys past the range masked; the online
    // softmax's reference update and O rescale; the weights P (bf16, and the
    // low parts for SPLIT_P); O^T += V^T . P^T with V from stage st.
    auto k_frags = [&](int st, bf16x8_t (&kf)[KS]) {
        const lds_char_t *ks = lsm + st * 2 * TILEB;
#pragma unroll
        for (int k = 0; k < KS; ++k) kf[k] = *(const bf16x8_t __attribute__((address_space(3))) *)(ks + kofs[k]);
    };
    auto qk = [&](const bf16x8_t (&kf)[KS]) {
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], sacc, 0, 0, 0);
        return sacc;
    };
    auto mask_tail = [&](f32x16_t &sacc, int t) {
        const int kt = k0 + t * NT;
        if (kt + NT > k1) {   // last tile of the range: mask keys past its end
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (kt + 16 * (j >> 3) + 8 * half + (j & 7) >= k1) sacc[j] = -INFINITY;
        }
    };
    auto rescale = [&](const f32x16_t &sacc) {
        // Online softmax along keys (one query row per lane, two lane halves).
        float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
        for (int j = 3; j < 16; j += 2) mx = fmaxf(fmaxf(mx, sacc[j]), sacc[j + 1 < 16 ? j + 1 : j]);
        mx = max_of_halves(mx) * c2;
        const bool grow = mx > m_run + kRescaleSlack;
        if (__any(grow)) {
            const float mnew = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
            m_run = mnew;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
    };
    auto probs = [&](const f32x16_t &sacc, uint32_t (&pk)[8], uint32_t (&pl)[8]) {
        const float nm = -m_run;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[j], c2, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[j + 1], c2, nm));
            bf16x2_t pp = {(__bf16)p0, (__bf16)p1};   // round to nearest even
            const uint32_t w = __builtin_bit_cast(uint32_t, pp);
            pk[j >> 1] = w;
            if constexpr (SPLIT_P) {
                bf16x2_t ll = {(__bf16)(p0 - bf16lo(w)), (__bf16)(p1 - bf16hi(w))};
                pl[j >> 1] = __builtin_bit_cast(uint32_t, ll);
                l_run += p0 + p1;
            } else {
                // Normalise by the weights the MFMA actually uses, so the
                // output stays a convex combination of V rows.
                l_run = fdot2(w, kOnesBf16x2, l_run);
            }
        }
    };
    auto pv = [&](const uint32_t (&pk)[8], const uint32_t (&pl)[8], int st) {
        const lds_char_t *vs = lsm + st * 2 * TILEB + TILEB;
        // O^T += V^T . P^T, two 16-key steps; V^T operands by transposing reads.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const u32x4_t pb = {pk[4 * kb + 0], pk[4 * kb + 1], pk[4 * kb + 2], pk[4 * kb + 3]};
            const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pb);
            const u32x4_t plb = {pl[4 * kb + 0], pl[4 * kb + 1], pl[4 * kb + 2], pl[4 * kb + 3]};
            const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, plb);
            const lds_char_t *vk = vs + kb * 16 * ROWB;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                typedef v4i16_t __attribute__((address_space(3))) *lds_v4i16_ptr;
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vk + vofs[db]));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vk + 4 * ROWB + vofs[db]));
                const u32x4_t w = {__builtin_bit_cast(u32x2_t, lo).x, __builtin_bit_cast(u32x2_t, lo).y,
                                   __builtin_bit_cast(u32x2_t, hi).x, __builtin_bit_cast(u32x2_t, hi).y};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pf, oacc[db], 0, 0, 0);
                if constexpr (SPLIT_P)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pfl, oacc[db], 0, 0, 0);
            }
        }
    };
    auto scores = [&](int st, int t) {
        bf16x8_t kf[KS];
        k_frags(st, kf);
        f32x16_t sacc = qk(kf);
        mask_tail(sacc, t);
        return sacc;
    };

    if constexpr (PIPE) {
        // Software-pipelined: tile t + 1's QK^T MFMAs are interleaved with
        // tile t's softmax weights (VALU and transcendental), so one wave's
        // matrix-core work overlaps its own VALU work (one prefix wave per SIMD
        // beside the paged pass).  At step t the wave needs tile t + 1 landed
        // (one tile less in flight), and the stage freed at step t still held
        // tile t - 1.  On the last step the K fragments come from a stage no
        // DMA writes any more and their scores are dropped.  A tile's keys
        // past the range are masked at the start of its own step.
        static_assert(PIPE == false || (KH == 1 && SWB && STAGES >= 4), "pipelined: one key half, deep ring");
        if (ntiles > STAGES - 2) wait_vmcnt<(STAGES - 2) * 2 * IPW>();   // tile 0; tiles 1 .. STAGES-2 in flight
        else wait_vmcnt<0>();
        waves_barrier(bar, (uint32_t)W * ++bar_k);
        f32x16_t s_cur;
        {
            bf16x8_t kf[KS];
            k_frags(0, kf);
            s_cur = qk(kf);               // masked at step 0
        }
        for (int t0 = 0; t0 < ntiles; t0 += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int t = t0 + st;
                if (t >= ntiles) break;
                const bool more = t + 1 < ntiles;
                if (more) {
                    // tile t + 1; tiles t + 2 .. t + STAGES - 2 issued after it
                    if (t + STAGES - 2 < ntiles) wait_vmcnt<(STAGES - 3) * 2 * IPW>();
                    else wait_vmcnt<0>();
                    waves_barrier(bar, (uint32_t)W * ++bar_k);   // every wave is done with tile t - 1
                    if (t + STAGES - 1 < ntiles) issue(t + STAGES - 1, (st + STAGES - 1) % STAGES);
                }
                bf16x8_t kf[KS];
                k_frags((st + 1) % STAGES, kf);
                // Branches (uniform) first, so that tile t's weights and tile
                // t + 1's MFMAs share one scheduling region.
                mask_tail(s_cur, t);
                rescale(s_cur);
                uint32_t pk[8], pl[8];
                probs(s_cur, pk, pl);
                f32x16_t s_nxt = qk(kf);
                // one MFMA of tile t + 1, then a few VALU of tile t's weights
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                pv(pk, pl, st);
                s_cur = s_nxt;
            }
        }
    } else {
        // Tile t sits in stage t % STAGES; the stage loop is unrolled so that all
        // LDS addresses are a per-lane offset plus an immediate.
        for (int t0 = 0; t0 < nt_loop; t0 += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int t = t0 + st;
                if (t >= nt_loop) break;
                const bool act = t < ntiles;   // this half still has tile t
                if (act) {
                    if (t + STAGES - 2 < ntiles) wait_vmcnt<AHEAD>();
                    else wait_vmcnt<0>();
                }
                if constexpr (SWB) {
                    waves_barrier(bar, (uint32_t)W * ++bar_k);
                } else {
                    __builtin_amdgcn_s_barrier();  // tile t visible; every wave is done with tile t-1
                    asm volatile("" ::: "memory");
                }
                if (!act) continue;
                if (t + STAGES - 1 < ntiles) issue(t + STAGES - 1, (st + STAGES - 1) % STAGES);
                f32x16_t sacc = scores(st, t);
                rescale(sacc);
                uint32_t pk[8], pl[8];
                probs(sacc, pk, pl);
                pv(pk, pl, st);
            }
        }
    }

    if constexpr (KH == 2) {
        // Half 1 hands its state (per lane: O^T registers, reference max and
        // normaliser) to the matching lane of half 0 through the ring's LDS.
        __builtin_amdgcn_s_barrier();          // every wave is done with both rings
        asm volatile("" ::: "memory");
        constexpr int NV = NDB * 16 + 2;
        float *xch = (float *)smem + (size_t)wave * NV * 64 + lane;
        if (khalf == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) xch[(db * 16 + j) * 64] = oacc[db][j];
            xch[(NV - 2) * 64] = m_run;
            xch[(NV - 1) * 64] = l_run;
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (khalf == 1) return;
        const float m1 = xch[(NV - 2) * 64], l1 = xch[(NV - 1) * 64];
        const float mt = fmaxf(m_run, m1);
        const float mu = mt == -INFINITY ? 0.f : mt;
        const float a0 = __builtin_amdgcn_exp2f(m_run - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] = oacc[db][j] * a0 + xch[(db * 16 + j) * 64] * a1;
        l_run = l_run * a0 + l1 * a1;
        m_run = mt;
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!row_ok) return;
    const int64_t prow = ((int64_t)qb * a.Hq + qj) * a.splits_total + s;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float *dst = a.o_part + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
            const int d = 32 * db + 8 * (j >> 2) + 4 * half;
            *(float4 *)(dst + d) = make_float4(oacc[db][j] * inv, oacc[db][j + 1] * inv, oacc[db][j + 2] * inv,
                                               oacc[db][j + 3] * inv);
        }
    if (half == 0) a.lse_part[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
}

template <int D, int W, bool SPLIT_P, int KH = 1>
__global__ __launch_bounds__(64 * W * KH) void prefix_mfma_kernel(Args a) {
    __shared__ __attribute__((aligned(1024))) char smem[prefix_ring_bytes<D, KH>()];
    __shared__ int32_t member_win[W * KH][kMemberWin];
    prefix_block<D, W, SPLIT_P, KH>(a, blockIdx.x, blockIdx.y, blockIdx.z,
                                    __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), smem, member_win);
}

// The paged pass and the prefix contraction in one launch (bf16, d = 128,
// prefix tiles of 2 or 4 row waves and two key halves): blocks
// [0, paged_blocks) are the paged pass's ranges (waves 0..3 of a block; the
// other four leave at once), the rest are prefix blocks (2 * PW waves).  Either role fills a CU's
// LDS, so one block runs per CU; blocks are handed out in index order, so
// every paged range starts at once (the split plan is one resident round)
// and prefix blocks take CUs as paged ranges finish: the prefix work fills
// the paged pass's tail and its own start-up overlaps the paged pass, with
// the same arithmetic and partial-state slots as the two separate launches.
// With fewer than 4 KV heads a paged block has hpb = 1 or 2 waves, and waves
// 0..3 of one launch block run 4 / hpb paged blocks side by side, each on its
// own rings: as many per CU as the paged plan counts.
// PW: row waves of the prefix tiles (4: all 8 waves of the block; 2: waves
// 0..3, the other four leave at once and are not waited for at barriers).
template <int D, int G, bool APP, bool NT, int PW>
__global__ __launch_bounds__(512) void paged_prefix_kernel(Args a, FlatLaunch fl, int paged_blocks, int psplits,
                                                           int pmtiles) {
    extern __shared__ __attribute__((aligned(1024))) char pp_smem[];
    const int bid = blockIdx.x;
    if (bid < paged_blocks) {
        const int wave = threadIdx.x >> 6;
        if (wave >= kFlatWavesMax) return;
        const int hpb = a.Hkv < kFlatWavesMax ? a.Hkv : kFlatWavesMax;   // 1, 2 or 4 (checked by the plan)
        const int per = kFlatWavesMax / hpb;                           // paged blocks per launch block
        const int pb = bid * per + wave / hpb;
        const int head_groups = (a.Hkv + hpb - 1) / hpb;
        if (pb >= fl.blocks * head_groups) return;
        const int sub = wave / hpb;
        flat_block<true, D, G, APP, NT>(a, fl, pb % fl.blocks, pb / fl.blocks, wave - sub * hpb, threadIdx.x & 63,
                                        pp_smem + sub * hpb * FlatMfmaGeom<D>::WAVEB);
        return;
    }
    if ((int)(threadIdx.x >> 6) >= 2 * PW) return;
    const int r = bid - paged_blocks;
    const int s = r % psplits, mt = (r / psplits) % pmtiles, gz = r / (psplits * pmtiles);
    prefix_block<D, PW, false, 2>(a, s, mt, gz, __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), pp_smem,
                                  (int32_t(*)[kMemberWin])(pp_smem + prefix_ring_bytes<D, 2>()));
}

// The paged pass and the prefix contraction side by side on every CU (bf16,
// d = 128): launch block b runs paged block b on waves 0..3 (rings of FS
// stages) and prefix item b on waves 4 .. 4 + PW - 1 (one key half, a ring of
// PS tiles).  The prefix waves meet at an LDS counter barrier of their own,
// so neither role waits for the other: the MFMA-bound contraction runs beside
// the HBM-bound paged pass instead of after it, with the same arithmetic and
// partial-state slots.  Both roles share the memory system, and each gets a
// share of its bandwidth in proportion to the bytes it keeps in flight, i.e.
// to its ring depth; the LDS holds FS = PS = 3, or FS = 2 and PS = 5 for
// plans whose prefix items have more key tiles than the paged waves have
// ring stages of tokens (the prefix role would finish last).
template <int FS, int PS>
constexpr size_t co_flat_bytes() { return (size_t)kFlatWavesMax * FlatMfmaGeom<128, FS>::WAVEB; }
template <int FS, int PS>
constexpr size_t co_lds() {
    return co_flat_bytes<FS, PS>() + prefix_ring_bytes<128, 1, PS>() + 4 * kMemberWin * sizeof(int32_t) + 16;
}
static_assert(co_flat_bytes<3, 3>() % 1024 == 0 && co_flat_bytes<2, 5>() % 1024 == 0,
              "the prefix ring starts 1 KB aligned");
static_assert(co_lds<3, 3>() <= (size_t)spkv::kLdsPerCU && co_lds<2, 5>() <= (size_t)spkv::kLdsPerCU,
              "one co-resident block per CU");

// Prefix item r of the co-resident launch, counted over cascade groups with a
// prefix only (group g holds nsplit_g * pmtiles * Hkv items, nsplit_g from
// the split rule), so that no launch block is left with an empty item while
// real ones wait for a second round.  One wave-wide pass over hot_len;
// returns false if r is past the last item.
__device__ __forceinline__ bool co_prefix_item(const Args &a, int r, int pmtiles, int &s, int &mt, int &gz) {
    const int lane = threadIdx.x & 63;
    int base = 0;                              // items of the groups before this 64-group window
    for (int g0 = 0; g0 < a.ng; g0 += 64) {
        const int g = g0 + lane;
        int n = 0;
        if (g < a.ng && mask_get(a.cascade, g)) {
            const int lp = a.hot_len[g];
            if (lp > 0) n = spkv::splits_for(lp, spkv::chunk_for(lp, a.prefix_tau, spkv::kPrefixSplitCap, a.prefix_granule));
        }
        const int c = n * pmtiles * a.Hkv;
        int incl = c;                          // inclusive prefix sum over the window's lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        const int total = __shfl(incl, 63, 64);
        if (r < base + total) {
            const uint64_t hit = __ballot(r < base + incl);
            const int gl = __builtin_ctzll(hit);   // first lane whose inclusive sum passes r
            const int ng_items = __shfl(n, gl, 64);
            const int local = r - base - (__shfl(incl, gl, 64) - __shfl(c, gl, 64));
            s = local % ng_items;
            mt = (local / ng_items) % pmtiles;
            gz = (g0 + gl) * a.Hkv + local / (ng_items * pmtiles);
            return true;
        }
        base += total;
    }
    return false;
}

template <int D, int G, bool APP, bool NT, int PW, int FS, int PS>
__global__ __launch_bounds__(512) void paged_prefix_co_kernel(Args a, FlatLaunch fl, int paged_blocks,
                                                              int prefix_items, int pmtiles) {
    static_assert(D == 128, "ring layout sized for d = 128");
    extern __shared__ __attribute__((aligned(1024))) char co_smem[];
    using F = FlatMfmaGeom<D, FS>;
    char *pring = co_smem + co_flat_bytes<FS, PS>();
    int32_t(*win)[kMemberWin] = (int32_t(*)[kMemberWin])(pring + prefix_ring_bytes<128, 1, PS>());
    uint32_t *bar = (uint32_t *)(win + 4);
    if (threadIdx.x == 0) *bar = 0u;
    __syncthreads();                           // every wave of the block is alive here
    const int bid = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    if (wave < kFlatWavesMax) {
        if (bid >= paged_blocks) return;
        const int hpb = a.Hkv < kFlatWavesMax ? a.Hkv : kFlatWavesMax;   // 1, 2 or 4 (checked by the plan)
        const int per = kFlatWavesMax / hpb;
        const int pb = bid * per + wave / hpb;
        const int head_groups = (a.Hkv + hpb - 1) / hpb;
        if (pb >= fl.blocks * head_groups) return;
        const int sub = wave / hpb;
        flat_block<true, D, G, APP, NT, FS>(a, fl, pb % fl.blocks, pb / fl.blocks, wave - sub * hpb,
                                            threadIdx.x & 63, co_smem + sub * hpb * F::WAVEB);
        return;
    }
    const int pw = wave - kFlatWavesMax;
    if (pw >= PW || bid >= prefix_items) return;
    int s = 0, mt = 0, gz = 0;
    if (!co_prefix_item(a, bid, pmtiles, s, mt, gz)) return;   // the same answer in every prefix wave
    s = __builtin_amdgcn_readfirstlane(s);     // wave-uniform already; say so for the scalar DMA bases
    mt = __builtin_amdgcn_readfirstlane(mt);
    gz = __builtin_amdgcn_readfirstlane(gz);
    prefix_block<D, PW, false, 1, PS, true, (PS >= 5)>(a, s, mt, gz, __builtin_amdgcn_readfirstlane(pw), pring, win,
                                                       bar);
}

// ---------------------------------------------------------------------------
// Prefix contraction for float32 pools ([GKV] Section 2.3: every member query
// of a group against the group's one slab), on the VALU in float32: a block of
// 256 threads takes 32 query rows of one group and KV head over one key chunk
// (the split rule of the bf16 contraction), with K / V tiles of 32 keys
// staged in LDS.  Eight consecutive lanes share a query row: each scores four
// keys of the tile and keeps D / 8 output dimensions; the row's online
// softmax state is reduced across those eight lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefix_f32_kernel(Args a) {
    constexpr int RT = 32;            // query rows per block
    constexpr int KT = 32;            // keys per tile
    constexpr int TPR = 8;            // lanes per row
    constexpr int KPT = KT / TPR;     // keys scored per lane per tile
    constexpr int DPT = D / TPR;      // output dims per lane
    constexpr int PAD = D + 4;        // LDS row stride in floats (rows start on distinct banks)
    constexpr int kWin = RT + 8;      // >= 32 rows / G + 1 members
    static_assert(spkv::kPrefixKeyTile == KT, "the split rule's granule is one tile");
    __shared__ float qs[RT][PAD];
    __shared__ float ks[KT][PAD];
    __shared__ float vs[KT][PAD];
    __shared__ float ps[RT][KT + 1];
    __shared__ int32_t win[kWin];
    __shared__ int32_t members_s;

    const int g = blockIdx.z / a.Hkv, h = blockIdx.z % a.Hkv;
    if (g >= a.ng || !mask_get(a.cascade, g)) return;
    const int64_t base = a.hot_base[g];
    const int lp = a.hot_len[g];
    if (lp <= 0 || base < 0 || base + lp > a.hot_capacity) return;
    const int mt = blockIdx.y;
    const int chunk = spkv::chunk_for(lp, a.prefix_tau, spkv::kPrefixSplitCap, KT);
    const int s = blockIdx.x;
    if (s >= spkv::splits_for(lp, chunk)) return;
    const int kc0 = s * chunk, kc1 = min(lp, kc0 + chunk);
    const int tid = threadIdx.x, lane = tid & 63;
    const int r = tid / TPR, kg = tid % TPR;

    // Members of group g (ascending request id, [GKV] Section 3.4): wave 0
    // scans group_of, counts them and writes the ids the block's rows need.
    const int kw0 = (mt * RT) / a.G;
    if (tid < 64) {
        int count = 0;
        for (int c0 = 0; c0 < a.B; c0 += 64) {
            const int i = c0 + lane;
            const bool mine = i < a.B && a.group_of[i] == g;
            const uint64_t m = __ballot(mine);
            const int rank = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (mine && rank >= kw0 && rank < kw0 + kWin) win[rank - kw0] = i;
            count += __popcll(m);
        }
        if (lane == 0) members_s = count;
    }
    __syncthreads();
    const int M = members_s * a.G;
    if (mt * RT >= M) return;                       // block-uniform

    const float *khot = (const float *)a.k_hot + slab_row(a, base, lp, h) * D;
    const float *vhot = (const float *)a.v_hot + slab_row(a, base, lp, h) * D;
    const int row = mt * RT + r;
    const bool row_ok = row < M;
    int qb = 0, qj = 0;
    if (row_ok) {
        qb = max(0, min(win[row / a.G - kw0], a.B - 1));
        qj = h * a.G + row % a.G;
    }
    // this row's query, D / 8 floats per lane, into LDS (zeros past the last row)
    {
        const float *qp = (const float *)a.q + ((int64_t)qb * a.Hq + qj) * D;
#pragma unroll
        for (int c = 0; c < DPT; c += 4) {
            const int col = kg * DPT + c;
            const float4 v = row_ok ? *(const float4 *)(qp + col) : make_float4(0.f, 0.f, 0.f, 0.f);
            *(float4 *)&qs[r][col] = v;
        }
    }
    float o[DPT];
#pragma unroll
    for (int c = 0; c < DPT; ++c) o[c] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;
    // The next tile's K / V pieces are loaded into registers while the
    // current tile is computed (one memory round trip per tile is hidden).
    constexpr int F4 = KT * D / 4;                  // float4 pieces of one tile
    constexpr int NPT = F4 / 256;                   // pieces per thread
    static_assert(F4 % 256 == 0, "a tile splits evenly over the block");
    float4 kpre[NPT], vpre[NPT];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int u = 0; u < NPT; ++u) {
            const int i = tid + 256 * u, key = i / (D / 4), c = (i % (D / 4)) * 4;
            const int64_t src = (int64_t)min(kt + key, kc1 - 1) * D + c;   // past the chunk: the last key (masked)
            kpre[u] = *(const float4 *)(khot + src);
            vpre[u] = *(const float4 *)(vhot + src);
        }
    };
    fetch(kc0);
    for (int kt = kc0; kt < kc1; kt += KT) {
        __syncthreads();                            // every lane is done with the previous tile
#pragma unroll
        for (int u = 0; u < NPT; ++u) {
            const int i = tid + 256 * u, key = i / (D / 4), c = (i % (D / 4)) * 4;
            *(float4 *)&ks[key][c] = kpre[u];
            *(float4 *)&vs[key][c] = vpre[u];
        }
        __syncthreads();
        if (kt + KT < kc1) fetch(kt + KT);
        float sc[KPT];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int key = kg + TPR * j;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; c += 4) {
                const float4 q4 = *(const float4 *)&qs[r][c];
                const float4 k4 = *(const float4 *)&ks[key][c];
                acc = fmaf(q4.x, k4.x, fmaf(q4.y, k4.y, fmaf(q4.z, k4.z, fmaf(q4.w, k4.w, acc))));
            }
            sc[j] = kt + key < kc1 ? acc * c2 : -INFINITY;
            mx = fmaxf(mx, sc[j]);
        }
        // the row's eight lanes are consecutive: reduce over aligned groups of 8
        mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const float pj = sc[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[j] - m_new);
            ps[r][kg + TPR * j] = pj;
            ls += pj;
        }
        ls += __shfl_xor(ls, 1, 64);
        ls += __shfl_xor(ls, 2, 64);
        ls += __shfl_xor(ls, 4, 64);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int c = 0; c < DPT; ++c) o[c] *= alpha;
        __builtin_amdgcn_wave_barrier();             // the row's weights (its own eight lanes) before they are read
        asm volatile("" ::: "memory");
        for (int key = 0; key < KT; ++key) {
            const float pk = ps[r][key];
#pragma unroll
            for (int c = 0; c < DPT; c += 4) {
                const float4 v4 = *(const float4 *)&vs[key][kg * DPT + c];
                o[c] = fmaf(pk, v4.x, o[c]);
                o[c + 1] = fmaf(pk, v4.y, o[c + 1]);
                o[c + 2] = fmaf(pk, v4.z, o[c + 2]);
                o[c + 3] = fmaf(pk, v4.w, o[c + 3]);
            }
        }
    }
    if (!row_ok) return;
    const int64_t prow = ((int64_t)qb * a.Hq + qj) * a.splits_total + s;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float *dst = a.o_part + prow * D + kg * DPT;
#pragma unroll
    for (int c = 0; c < DPT; c += 4)
        *(float4 *)(dst + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
    if (kg == 0) a.lse_part[prow] = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Merge of a row's partial states (Eq. (1) applied across all partials).
// One wave per (request, query head) row; four rows per block.  Each
// wave-wide load brings PPW partial rows (LPP lanes x 16 bytes each), several
// loads in flight; every lane keeps an online merge of the partials it reads.
// ---------------------------------------------------------------------------
// APPEND: the merge launch also lands the step's new tokens, which the paged
// pass read from k_new / v_new: every reader of the pools, block tables and
// lengths has finished by now (same stream), so extra blocks copy each
// request's K/V rows into its slot and advance its block table and length,
// as spkv_append_tokens does.
// Kernel arguments are limited to 4 KB; the by-value tables are sized so the
// largest argument lists (the merge's, the paged launches') stay within it.
struct MergeKernargs { Args a; float *out, *lse; FlatLaunch fr; MergeRows ap; };
struct PagedKernargs { Args a; FlatLaunch fl; int x, y, z; };
static_assert(sizeof(MergeKernargs) <= 4096, "merge kernel arguments exceed 4 KB");
static_assert(sizeof(PagedKernargs) <= 4096, "paged-pass kernel arguments exceed 4 KB");

template <int D, bool APPEND = false>
__global__ __launch_bounds__(256) void merge_kernel(Args a, float *out, float *lse_out, FlatLaunch fr,
                                                    MergeRows ap) {
    constexpr int LPP = D / 4;      // lanes per partial row (float4 each)
    constexpr int PPW = 64 / LPP;   // partial rows per wave-wide load
    constexpr int BATCH = 40 / PPW; // wave-wide loads in flight (40 partials)
    constexpr int MID = 24 / PPW;   // the same for rows of at most 24 partials,
    constexpr int SMALL = 16 / PPW; // 16
    constexpr int TINY = 8 / PPW;   // and 8
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: geometry by scalar loads
    const int lane = threadIdx.x & 63;
    if constexpr (APPEND) {
        // Blocks past the merge's own land the new tokens, one wave per
        // request, beside the merging waves: each copies the request's K/V
        // rows into its slot and advances its block table and length.  Every
        // reader of these (the paged pass; this kernel reads none) is done.
        const int64_t merge_blocks = ((int64_t)fr.nreq * a.Hq + 3) / 4;
        if ((int64_t)blockIdx.x >= merge_blocks) {
            const int i = (int)(((int64_t)blockIdx.x - merge_blocks) * 4 + wave);
            if (i >= fr.nreq) return;
            const int b = fr.b0 + i;
            const int64_t slot = ap.slots[i];
            const int pieces = a.Hkv * D * 2 / 16;   // 16-byte pieces of one token's K (or V) row
            const u32x4_t *kn = (const u32x4_t *)a.k_new + (int64_t)b * pieces;
            const u32x4_t *vn = (const u32x4_t *)a.v_new + (int64_t)b * pieces;
            u32x4_t *kc = (u32x4_t *)a.k_cold + slot * pieces;
            u32x4_t *vc = (u32x4_t *)a.v_cold + slot * pieces;
            for (int q = lane; q < pieces; q += 64) {
                kc[q] = kn[q];
                vc[q] = vn[q];
            }
            if (lane == 0) {
                int32_t *lens = (int32_t *)a.cold_lens;
                const int len = lens[b];
                ((int32_t *)a.tables)[(int64_t)b * a.max_blocks + len / a.page_size] = (int32_t)(slot / a.page_size);
                lens[b] = len + 1;
            }
            return;
        }
    }
    const int64_t row = (int64_t)fr.b0 * a.Hq + (int64_t)blockIdx.x * 4 + wave;
    if (row >= (int64_t)(fr.b0 + fr.nreq) * a.Hq) return;
    const int b = (int)(row / a.Hq);
    const int i = b - fr.b0;
    int np = a.prefix_mode == 1 ? ap.prefix_np[i] : 0;
    int nf = ap.flat_np[i];
    np = max(0, min(np, a.prefix_splits));   // never read past this row's partial slots
    nf = max(0, min(nf, a.flat_splits));
    const int n = np + nf;           // <= 128
    const int64_t prow0 = row * a.splits_total;
    auto slot_of = [&](int k) { return k < np ? k : a.prefix_splits + (k - np); };
    if (n == 0) {                    // empty context: zero output, log-sum-exp -inf
        if (lane < D / 4) *(float4 *)(out + row * D + lane * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lse_out && lane == 0) lse_out[row] = -INFINITY;
        return;
    }

    const int sub = lane % LPP;      // float4 column of the row
    const int which = lane / LPP;    // partial within a wave-wide load
    // Row base (wave-uniform) plus a 32-bit byte offset per lane.
    const char *prow_base = (const char *)(a.o_part + prow0 * D);
    auto part_ptr = [&](int k) {
        return (const f32x4v_t *)(prow_base + (uint32_t)(slot_of(k) * (D * 4) + sub * 16));
    };

    // Each lane reads the log-sum-exp of the partials whose rows it reads, so
    // its weights need no cross-lane step: a batch is one round of loads (the
    // partial rows and their log-sum-exps together), a running maximum per
    // lane, and FMAs; the LPP-lane groups that read different partials merge
    // their states once at the end (Eq. (1) between lanes).  Loads past the
    // last partial re-read partial 0 (in bounds; weight 0), so a batch is
    // straight-line code with a single wait; a row takes the smallest batch
    // that holds its partials (loads that only re-read partial 0 still cost).  (Non-temporal: partial states are read once, and must
    // not displace K/V lines the next step reads again.)
    const float *lrow = a.lse_part + prow0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float mx = -INFINITY, wsum = 0.f;
    auto run = [&](auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        f32x4v_t v[NB];
        float lk[NB];
        for (int k0 = 0; k0 < n; k0 += PPW * NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int k = k0 + u * PPW + which;
                const int kk = k < n ? k : 0;
                v[u] = __builtin_nontemporal_load(part_ptr(kk));
                lk[u] = __builtin_nontemporal_load(lrow + slot_of(kk));
            }
            float bm = -INFINITY;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                if (k0 + u * PPW + which >= n) lk[u] = -INFINITY;
                bm = fmaxf(bm, lk[u]);
            }
            const float nm = fmaxf(mx, bm);
            const float muse = nm == -INFINITY ? 0.f : nm;
            const float sc = exp2f(mx - muse);   // 0 while mx is -inf
            acc.x *= sc;
            acc.y *= sc;
            acc.z *= sc;
            acc.w *= sc;
            wsum *= sc;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const float w = exp2f(lk[u] - muse);
                acc.x = fmaf(w, v[u].x, acc.x);
                acc.y = fmaf(w, v[u].y, acc.y);
                acc.z = fmaf(w, v[u].z, acc.z);
                acc.w = fmaf(w, v[u].w, acc.w);
                wsum += w;
            }
            mx = nm;
        }
    };
    if (n <= PPW * TINY) run(std::integral_constant<int, TINY>{});
    else if (n <= PPW * SMALL) run(std::integral_constant<int, SMALL>{});
    else if (n <= PPW * MID) run(std::integral_constant<int, MID>{});
    else run(std::integral_constant<int, BATCH>{});
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) {
        const float om = __shfl_xor(mx, off, 64);
        const float ow = __shfl_xor(wsum, off, 64);
        const float ox = __shfl_xor(acc.x, off, 64), oy = __shfl_xor(acc.y, off, 64);
        const float oz = __shfl_xor(acc.z, off, 64), ov = __shfl_xor(acc.w, off, 64);
        const float nm = fmaxf(mx, om);
        const float muse = nm == -INFINITY ? 0.f : nm;
        const float s0 = exp2f(mx - muse), s1 = exp2f(om - muse);
        acc.x = acc.x * s0 + ox * s1;
        acc.y = acc.y * s0 + oy * s1;
        acc.z = acc.z * s0 + oz * s1;
        acc.w = acc.w * s0 + ov * s1;
        wsum = wsum * s0 + ow * s1;
        mx = nm;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (which == 0)
        *(float4 *)(out + row * D + sub * 4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (lse_out && lane == 0) lse_out[row] = wsum > 0.f ? (mx + __log2f(wsum)) * kLn2 : -INFINITY;
}

// Two-way merge of natural-log partial states, Eq. (1).  head_dim divides the
// block size, so a row never straddles blocks; all reads of a block finish
// before any write, which makes in-place use (o == o_a, lse == lse_a) safe.
__global__ __launch_bounds__(256) void merge2_kernel(const float *oa, const float *la, const float *ob, const float *lb,
                                                     float *o, float *lse, int64_t rows, int d) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool ok = i < rows * d;
    const int64_t r = ok ? i / d : 0;
    float wa = 0.f, wb = 0.f, va = 0.f, vb = 0.f, mu = 0.f;
    if (ok) {
        const float xa = la[r], xb = lb[r];
        const float m = fmaxf(xa, xb);
        mu = m == -INFINITY ? 0.f : m;
        wa = expf(xa - mu);
        wb = expf(xb - mu);
        va = oa[i];
        vb = ob[i];
    }
    __syncthreads();
    if (!ok) return;
    const float w = wa + wb;
    o[i] = w > 0.f ? (wa * va + wb * vb) / w : 0.f;
    if (lse && i % d == 0) lse[r] = w > 0.f ? mu + logf(w) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Cache writes: 16-byte copies.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hot_write_kernel(const u32x4_t *ksrc, const u32x4_t *vsrc, u32x4_t *khot,
                                                        u32x4_t *vhot, int64_t base, int64_t lp, int num_layers, int layer,
                                                        int hkv, int pieces_per_row) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = lp * hkv * pieces_per_row;
    if (i >= total) return;
    const int64_t piece = i % pieces_per_row;
    const int64_t th = i / pieces_per_row;      // token-major source row: t * hkv + h
    const int64_t t = th / hkv;
    const int64_t h = th % hkv;
    const int64_t dst = ((base * hkv * num_layers + (int64_t)layer * lp * hkv + h * lp) + t) * pieces_per_row + piece;
    khot[dst] = ksrc[i];
    vhot[dst] = vsrc[i];
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const u32x4_t *knew, const u32x4_t *vnew,
                                                                const int32_t *slots, int n, u32x4_t *kcold,
                                                                u32x4_t *vcold, int64_t cold_slots, int pieces_per_slot) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n * pieces_per_slot) return;
    const int64_t tok = i / pieces_per_slot;
    const int64_t piece = i % pieces_per_slot;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= cold_slots) return;
    kcold[slot * pieces_per_slot + piece] = knew[i];
    vcold[slot * pieces_per_slot + piece] = vnew[i];
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t *pairs, u32x4_t *kcold, u32x4_t *vcold,
                                                          int num_pages, int64_t pieces_per_page) {
    const int p = blockIdx.y;
    const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_pages || dst < 0 || dst >= num_pages) return;
    const int64_t layer_off = (int64_t)blockIdx.z * num_pages * pieces_per_page;   // layer of the pool
    kcold += layer_off;
    vcold += layer_off;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces_per_page; i += (int64_t)gridDim.x * blockDim.x) {
        kcold[dst * pieces_per_page + i] = kcold[src * pieces_per_page + i];
        vcold[dst * pieces_per_page + i] = vcold[src * pieces_per_page + i];
    }
}

__global__ __launch_bounds__(256) void block_table_append_kernel(int32_t *tables, int max_blocks, int32_t *lens,
                                                                 int num_rows, const int32_t *rows,
                                                                 const int32_t *slots, int n, int page_size) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int r = rows[i];
    if (r < 0 || r >= num_rows) return;
    const int len = lens[r];
    const int blk = len / page_size;
    if (len < 0 || blk >= max_blocks) return;
    tables[(int64_t)r * max_blocks + blk] = slots[i] / page_size;
    lens[r] = len + 1;
}

// One decode step's appends in one launch: token i's K and V rows go to COLD
// slot slots[i], and request rows[i]'s device block table and length follow
// the append.  Slots and rows arrive from the host allocator through the
// kernel arguments (no upload); block x handles token x.
constexpr int kAppendArgTokens = 256;
struct AppendArgs {
    int32_t n;
    int32_t slots[kAppendArgTokens];
    int32_t rows[kAppendArgTokens];
};
static_assert(sizeof(AppendArgs) + 10 * sizeof(void *) <= 4096, "append kernel arguments exceed 4 KB");

__global__ __launch_bounds__(256) void append_tokens_kernel(const u32x4_t *knew, const u32x4_t *vnew, AppendArgs aa,
                                                            u32x4_t *kcold, u32x4_t *vcold, int64_t cold_slots,
                                                            int pieces_per_slot, int32_t *tables, int max_blocks,
                                                            int32_t *lens, int num_rows, int page_size) {
    const int tok = blockIdx.x;
    if (tok >= aa.n) return;
    const int64_t slot = aa.slots[tok];
    if (slot < 0 || slot >= cold_slots) return;
    for (int p = threadIdx.x; p < pieces_per_slot; p += blockDim.x) {
        kcold[slot * pieces_per_slot + p] = knew[(int64_t)tok * pieces_per_slot + p];
        vcold[slot * pieces_per_slot + p] = vnew[(int64_t)tok * pieces_per_slot + p];
    }
    if (threadIdx.x == 0 && tables) {
        const int r = aa.rows[tok];
        if (r < 0 || r >= num_rows) return;
        const int len = lens[r];
        const int blk = len / page_size;
        if (len < 0 || blk >= max_blocks) return;
        tables[(int64_t)r * max_blocks + blk] = (int32_t)(slot / page_size);
        lens[r] = len + 1;
    }
}

// ---------------------------------------------------------------------------
// Launch plumbing and optional per-launch timing.
// ---------------------------------------------------------------------------
struct Timing {
    std::mutex mu;
    bool on = false;
    struct Rec { int kernel; hipEvent_t a, b; };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double total_ms[SPKV_NUM_KERNELS] = {};
    int64_t count[SPKV_NUM_KERNELS] = {};
};
Timing &timing() {
    static Timing t;
    return t;
}

hipEvent_t take_event(Timing &t) {
    if (!t.pool.empty()) {
        hipEvent_t e = t.pool.back();
        t.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// With timing on, a launch goes through hipExtLaunchKernelGGL with a start and
// a stop event: the events take the dispatch's own begin and end timestamps,
// so no marker packet sits between two kernels of the stream and the duration
// is the kernel's alone.  Otherwise it is a plain launch.
struct TimedLaunch {
    int kernel;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    bool used = false;
    TimedLaunch(int k, hipStream_t s) : kernel(k), st(s) {
        Timing &t = timing();
        std::lock_guard<std::mutex> g(t.mu);
        if (!t.on) return;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone) return;   // a graph node: no events
        a = take_event(t);
        b = take_event(t);
    }
    template <typename... P, typename... V>
    void launch(void (*kern)(P...), dim3 grid, dim3 block, size_t lds, V... args) {
        if (a && b) {
            hipExtLaunchKernelGGL(kern, grid, block, (std::uint32_t)lds, st, a, b, 0u, args...);
            used = true;
        } else {
            kern<<<grid, block, lds, st>>>(args...);
        }
    }
    ~TimedLaunch() {
        Timing &t = timing();
        std::lock_guard<std::mutex> g(t.mu);
        if (a && b && used) {
            t.pending.push_back({kernel, a, b});
            return;
        }
        if (a) t.pool.push_back(a);
        if (b) t.pool.push_back(b);
    }
};

spkv_status check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return SPKV_OK;
}

// Dynamic LDS above 64 KB is granted per kernel once its limit is raised.
template <bool BF16, int D, int G, bool APP, bool NT>
spkv_status launch_flat_k(const Args &a, const FlatLaunch &f, dim3 grid, dim3 block, size_t lds,
                          TimedLaunch &tl) {
    static const hipError_t attr = hipFuncSetAttribute((const void *)flat_kernel<BF16, D, G, APP, NT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, spkv::kLdsPerCU);
    if (attr != hipSuccess) return fail(SPKV_E_HIP, std::string("flat_kernel LDS limit: ") + hipGetErrorString(attr));
    tl.launch(flat_kernel<BF16, D, G, APP, NT>, grid, block, lds, a, f);
    return check_launch("flat_kernel");
}

// bf16: append mode (the step's new tokens come from k_new / v_new) and the
// streaming hint select the instantiation.
template <bool BF16, int D, int G>
spkv_status launch_flat_g(const Args &a, const FlatLaunch &f, dim3 grid, dim3 block, size_t lds,
                          const int32_t *append_slots, TimedLaunch &tl) {
    if constexpr (BF16) {
        if (append_slots)
            return a.cold_nt ? launch_flat_k<BF16, D, G, true, true>(a, f, grid, block, lds, tl)
                             : launch_flat_k<BF16, D, G, true, false>(a, f, grid, block, lds, tl);
        if (a.cold_nt) return launch_flat_k<BF16, D, G, false, true>(a, f, grid, block, lds, tl);
    }
    return launch_flat_k<BF16, D, G, false, false>(a, f, grid, block, lds, tl);
}

template <bool BF16, int D>
spkv_status launch_flat_d(const Args &a, const FlatLaunch &f, int head_groups,
                          const int32_t *append_slots, hipStream_t st) {
    const int waves = a.Hkv < kFlatWavesMax ? a.Hkv : kFlatWavesMax;
    dim3 grid(f.blocks, head_groups), block(64 * waves);
    const size_t lds = (size_t)waves * (BF16 ? FlatMfmaGeom<D>::WAVEB : FlatGeom<BF16, D>::WAVEB);
    TimedLaunch tl(SPKV_KERNEL_FLAT, st);
    switch (a.G) {
    case 1: return launch_flat_g<BF16, D, 1>(a, f, grid, block, lds, append_slots, tl);
    case 2: return launch_flat_g<BF16, D, 2>(a, f, grid, block, lds, append_slots, tl);
    case 3: return launch_flat_g<BF16, D, 3>(a, f, grid, block, lds, append_slots, tl);
    case 4: return launch_flat_g<BF16, D, 4>(a, f, grid, block, lds, append_slots, tl);
    case 5: return launch_flat_g<BF16, D, 5>(a, f, grid, block, lds, append_slots, tl);
    case 6: return launch_flat_g<BF16, D, 6>(a, f, grid, block, lds, append_slots, tl);
    case 7: return launch_flat_g<BF16, D, 7>(a, f, grid, block, lds, append_slots, tl);
    case 8: return launch_flat_g<BF16, D, 8>(a, f, grid, block, lds, append_slots, tl);
    default: return fail(SPKV_E_INVAL, "unsupported GQA group size");
    }
}

spkv_status launch_flat(const Args &a, bool bf16, int d, const FlatLaunch &f, int head_groups,
                        const int32_t *append_slots, hipStream_t st) {
    if (f.blocks <= 0 || a.B == 0) return SPKV_OK;
    if (bf16) return d == 128 ? launch_flat_d<true, 128>(a, f, head_groups, append_slots, st)
                              : launch_flat_d<true, 64>(a, f, head_groups, append_slots, st);
    return d == 128 ? launch_flat_d<false, 128>(a, f, head_groups, nullptr, st)
                    : launch_flat_d<false, 64>(a, f, head_groups, nullptr, st);
}

spkv_status launch_prefix(const Args &a, const Plan &p, int d, bool bf16, hipStream_t st) {
    if (p.prefix_splits <= 0 || p.prefix_mtiles <= 0) return SPKV_OK;
    if (!bf16) {
        dim3 grid(p.prefix_splits, p.prefix_mtiles, a.ng * a.Hkv), block(256);
        TimedLaunch tl(SPKV_KERNEL_PREFIX, st);
        if (d == 128) tl.launch(prefix_f32_kernel<128>, grid, block, 0, a);
        else tl.launch(prefix_f32_kernel<64>, grid, block, 0, a);
        return check_launch("prefix_f32_kernel");
    }
    dim3 grid(p.prefix_splits, p.prefix_mtiles, a.ng * a.Hkv), block(64 * p.prefix_waves * p.prefix_key_halves);
    TimedLaunch tl(SPKV_KERNEL_PREFIX, st);
    const int key = p.prefix_waves * 1000 + d + (p.prefix_split_p ? 10000 : 0) + (p.prefix_key_halves == 2 ? 100000 : 0);
    switch (key) {
    case 104128: tl.launch(prefix_mfma_kernel<128, 4, false, 2>, grid, block, 0, a); break;
    case 102128: tl.launch(prefix_mfma_kernel<128, 2, false, 2>, grid, block, 0, a); break;
    case 102064: tl.launch(prefix_mfma_kernel<64, 2, false, 2>, grid, block, 0, a); break;
    case 112128: tl.launch(prefix_mfma_kernel<128, 2, true, 2>, grid, block, 0, a); break;
    case 112064: tl.launch(prefix_mfma_kernel<64, 2, true, 2>, grid, block, 0, a); break;
    case 104064: tl.launch(prefix_mfma_kernel<64, 4, false, 2>, grid, block, 0, a); break;
    case 114128: tl.launch(prefix_mfma_kernel<128, 4, true, 2>, grid, block, 0, a); break;
    case 114064: tl.launch(prefix_mfma_kernel<64, 4, true, 2>, grid, block, 0, a); break;
    case 1128: tl.launch(prefix_mfma_kernel<128, 1, false>, grid, block, 0, a); break;
    case 2128: tl.launch(prefix_mfma_kernel<128, 2, false>, grid, block, 0, a); break;
    case 4128: tl.launch(prefix_mfma_kernel<128, 4, false>, grid, block, 0, a); break;
    case 1064: tl.launch(prefix_mfma_kernel<64, 1, false>, grid, block, 0, a); break;
    case 2064: tl.launch(prefix_mfma_kernel<64, 2, false>, grid, block, 0, a); break;
    case 4064: tl.launch(prefix_mfma_kernel<64, 4, false>, grid, block, 0, a); break;
    case 11128: tl.launch(prefix_mfma_kernel<128, 1, true>, grid, block, 0, a); break;
    case 12128: tl.launch(prefix_mfma_kernel<128, 2, true>, grid, block, 0, a); break;
    case 14128: tl.launch(prefix_mfma_kernel<128, 4, true>, grid, block, 0, a); break;
    case 11064: tl.launch(prefix_mfma_kernel<64, 1, true>, grid, block, 0, a); break;
    case 12064: tl.launch(prefix_mfma_kernel<64, 2, true>, grid, block, 0, a); break;
    case 14064: tl.launch(prefix_mfma_kernel<64, 4, true>, grid, block, 0, a); break;
    default: return fail(SPKV_E_INVAL, "unsupported prefix tile");
    }
    return check_launch("prefix_mfma_kernel");
}

// LDS of one paged_prefix_kernel block: the larger of the paged pass's four
// rings and the prefix block's two rings plus its member windows.
constexpr size_t paged_prefix_lds() {
    constexpr size_t paged = (size_t)kFlatWavesMax * FlatMfmaGeom<128>::WAVEB;
    constexpr size_t prefix = (size_t)prefix_ring_bytes<128, 2>() + 8 * kMemberWin * sizeof(int32_t);
    return paged > prefix ? paged : prefix;
}
static_assert(paged_prefix_lds() <= (size_t)spkv::kLdsPerCU, "one paged_prefix_kernel block per CU");
static_assert(2 * paged_prefix_lds() > (size_t)spkv::kLdsPerCU, "one launch block per CU, as the plan counts");

template <int G, bool APP, bool NT, int PW>
spkv_status launch_paged_prefix_k(const Args &a, const Plan &p, TimedLaunch &tl) {
    constexpr int D = 128;
    static const hipError_t attr = hipFuncSetAttribute((const void *)paged_prefix_kernel<D, G, APP, NT, PW>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, spkv::kLdsPerCU);
    if (attr != hipSuccess) return fail(SPKV_E_HIP, std::string("paged_prefix_kernel LDS limit: ") + hipGetErrorString(attr));
    const FlatLaunch &f = p.flat[0];
    const int hpb = a.Hkv < kFlatWavesMax ? a.Hkv : kFlatWavesMax;
    const int per = kFlatWavesMax / hpb;
    const int64_t paged = ((int64_t)f.blocks * p.flat_head_groups + per - 1) / per;
    const int64_t prefix = (int64_t)p.prefix_splits * p.prefix_mtiles * a.ng * a.Hkv;
    if (paged + prefix >= ((int64_t)1 << 31)) return fail(SPKV_E_INVAL, "paged_prefix_kernel: grid too large");
    dim3 grid((unsigned)(paged + prefix)), block(512);
    tl.launch(paged_prefix_kernel<D, G, APP, NT, PW>, grid, block, paged_prefix_lds(), a, f, (int)paged,
              p.prefix_splits, p.prefix_mtiles);
    return check_launch("paged_prefix_kernel");
}

template <int G, int PW>
spkv_status launch_paged_prefix_w(const Args &a, const Plan &p, bool app, TimedLaunch &tl) {
    if (app) return a.cold_nt ? launch_paged_prefix_k<G, true, true, PW>(a, p, tl)
                              : launch_paged_prefix_k<G, true, false, PW>(a, p, tl);
    return a.cold_nt ? launch_paged_prefix_k<G, false, true, PW>(a, p, tl)
                     : launch_paged_prefix_k<G, false, false, PW>(a, p, tl);
}

template <int G>
spkv_status launch_paged_prefix_g(const Args &a, const Plan &p, bool app, TimedLaunch &tl) {
    return p.prefix_waves == 4 ? launch_paged_prefix_w<G, 4>(a, p, app, tl) : launch_paged_prefix_w<G, 2>(a, p, app, tl);
}

template <int G, bool APP, bool NT, int PW, int FS, int PS>
spkv_status launch_paged_prefix_co_k(const Args &a, const Plan &p, TimedLaunch &tl) {
    constexpr int D = 128;
    static const hipError_t attr = hipFuncSetAttribute((const void *)paged_prefix_co_kernel<D, G, APP, NT, PW, FS, PS>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, spkv::kLdsPerCU);
    if (attr != hipSuccess)
        return fail(SPKV_E_HIP, std::string("paged_prefix_co_kernel LDS limit: ") + hipGetErrorString(attr));
    const FlatLaunch &f = p.flat[0];
    const int hpb = a.Hkv < kFlatWavesMax ? a.Hkv : kFlatWavesMax;
    const int per = kFlatWavesMax / hpb;
    const int64_t paged = ((int64_t)f.blocks * p.flat_head_groups + per - 1) / per;
    const int64_t prefix = p.co_prefix_items;
    if (paged >= ((int64_t)1 << 31) || prefix >= ((int64_t)1 << 31))
        return fail(SPKV_E_INVAL, "paged_prefix_co_kernel: grid too large");
    dim3 grid((unsigned)std::max(paged, prefix)), block(512);
    tl.launch(paged_prefix_co_kernel<D, G, APP, NT, PW, FS, PS>, grid, block, co_lds<FS, PS>(), a, f, (int)paged,
              (int)prefix, p.prefix_mtiles);
    return check_launch("paged_prefix_co_kernel");
}

template <int G, int PW, int FS, int PS>
spkv_status launch_paged_prefix_co_w(const Args &a, const Plan &p, bool app, TimedLaunch &tl) {
    if (app) return a.cold_nt ? launch_paged_prefix_co_k<G, true, true, PW, FS, PS>(a, p, tl)
                              : launch_paged_prefix_co_k<G, true, false, PW, FS, PS>(a, p, tl);
    return a.cold_nt ? launch_paged_prefix_co_k<G, false, true, PW, FS, PS>(a, p, tl)
                     : launch_paged_prefix_co_k<G, false, false, PW, FS, PS>(a, p, tl);
}

// The deep prefix ring (FS = 2, PS = 5) for tiles of 4 row waves only, the
// shape whose contraction can outlast the paged pass.
template <int G>
spkv_status launch_paged_prefix_co_g(const Args &a, const Plan &p, bool app, TimedLaunch &tl) {
    if (p.prefix_waves != 4) return launch_paged_prefix_co_w<G, 2, 3, 3>(a, p, app, tl);
    return p.co_prefix_stages == 5 ? launch_paged_prefix_co_w<G, 4, 2, 5>(a, p, app, tl)
                                   : launch_paged_prefix_co_w<G, 4, 3, 3>(a, p, app, tl);
}

spkv_status launch_paged_prefix_co(const Args &a, const Plan &p, bool app, hipStream_t st) {
    TimedLaunch tl(SPKV_KERNEL_PAGED_PREFIX, st);
    switch (a.G) {
    case 1: return launch_paged_prefix_co_g<1>(a, p, app, tl);
    case 2: return launch_paged_prefix_co_g<2>(a, p, app, tl);
    case 3: return launch_paged_prefix_co_g<3>(a, p, app, tl);
    case 4: return launch_paged_prefix_co_g<4>(a, p, app, tl);
    case 5: return launch_paged_prefix_co_g<5>(a, p, app, tl);
    case 6: return launch_paged_prefix_co_g<6>(a, p, app, tl);
    case 7: return launch_paged_prefix_co_g<7>(a, p, app, tl);
    case 8: return launch_paged_prefix_co_g<8>(a, p, app, tl);
    default: return fail(SPKV_E_INVAL, "paged_prefix_co_kernel: unsupported group size");
    }
}

spkv_status launch_paged_prefix(const Args &a, const Plan &p, bool app, hipStream_t st) {
    TimedLaunch tl(SPKV_KERNEL_PAGED_PREFIX, st);
    switch (a.G) {
    case 1: return launch_paged_prefix_g<1>(a, p, app, tl);
    case 2: return launch_paged_prefix_g<2>(a, p, app, tl);
    case 3: return launch_paged_prefix_g<3>(a, p, app, tl);
    case 4: return launch_paged_prefix_g<4>(a, p, app, tl);
    case 5: return launch_paged_prefix_g<5>(a, p, app, tl);
    case 6: return launch_paged_prefix_g<6>(a, p, app, tl);
    case 7: return launch_paged_prefix_g<7>(a, p, app, tl);
    case 8: return launch_paged_prefix_g<8>(a, p, app, tl);
    default: return fail(SPKV_E_INVAL, "unsupported GQA group size");
    }
}

spkv_status launch_merge(const Args &a, int d, float *out, float *lse, const FlatLaunch &fr,
                         const int32_t *append_slots, const uint8_t *prefix_np, hipStream_t st) {
    const int64_t rows = (int64_t)fr.nreq * a.Hq;
    if (rows == 0) return SPKV_OK;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    TimedLaunch tl(SPKV_KERNEL_MERGE, st);
    MergeRows ap{};
    if (prefix_np)
        for (int i = 0; i < fr.nreq; ++i) ap.prefix_np[i] = prefix_np[fr.b0 + i];
    for (int i = 0; i < fr.nreq; ++i) {
        int first;
        ap.flat_np[i] = (uint8_t)std::min(flat_parts(fr, i, &first), 255);
    }
    if (append_slots) {
        for (int i = 0; i < fr.nreq; ++i) ap.slots[i] = append_slots[fr.b0 + i];
        grid.x += (unsigned)((fr.nreq + 3) / 4);   // the new-token waves
        if (d == 128) tl.launch(merge_kernel<128, true>, grid, block, 0, a, out, lse, fr, ap);
        else tl.launch(merge_kernel<64, true>, grid, block, 0, a, out, lse, fr, ap);
    } else {
        if (d == 128) tl.launch(merge_kernel<128>, grid, block, 0, a, out, lse, fr, ap);
        else tl.launch(merge_kernel<64>, grid, block, 0, a, out, lse, fr, ap);
    }
    return check_launch("merge_kernel");
}

Args make_args(const spkv_batch *b, const spkv_kv *kv, const Plan &p, void *ws) {
    Args a;
    std::memset(&a, 0, sizeof(a));
    a.q = b->q;
    a.B = b->batch;
    a.Hq = b->num_q_heads;
    a.Hkv = b->num_kv_heads;
    a.G = b->num_q_heads / b->num_kv_heads;
    a.scale_log2 = b->scale * kLog2e;
    a.ng = b->num_groups;
    a.group_of = b->group_of;
    a.hot_base = b->hot_base;
    a.hot_len = b->hot_len;
    a.page_size = b->page_size;
    a.max_blocks = b->max_blocks;
    a.tables = b->block_tables;
    a.cold_lens = b->cold_lens;
    a.k_hot = kv->k_hot;
    a.v_hot = kv->v_hot;
    a.hot_capacity = kv->hot_capacity;
    a.num_layers = kv->num_layers;
    a.layer = kv->layer;
    const int64_t cold_layer = (int64_t)kv->layer * kv->cold_slots * b->num_kv_heads * b->head_dim *
                               (b->dtype == SPKV_DTYPE_BF16 ? 2 : 4);
    a.k_cold = kv->k_cold ? (const char *)kv->k_cold + cold_layer : nullptr;
    a.v_cold = kv->v_cold ? (const char *)kv->v_cold + cold_layer : nullptr;
    a.cold_slots = kv->cold_slots;
    const int64_t rows = (int64_t)b->batch * b->num_q_heads;
    a.o_part = (float *)ws;
    a.lse_part = (float *)((char *)ws + ((rows * p.splits_total * b->head_dim * 4 + 255) / 256) * 256);
    a.splits_total = p.splits_total;
    a.prefix_splits = p.prefix_splits;
    a.flat_splits = p.flat_splits;
    a.flat_tau = p.flat_chunk;
    a.prefix_tau = p.prefix_chunk > 0 ? p.prefix_chunk : 1;
    a.prefix_granule = spkv::kPrefixKeyTile;
    a.prefix_mode = p.run_prefix ? 1 : 0;
    a.cascade = p.cascade;
    return a;
}

// The step's new tokens, in append mode (spkv_decode_step_append).
struct AppendIn {
    const void *k_new;
    const void *v_new;
    const int32_t *slots;   // host [B]
};

// single_launch: where the plan allows one launch for the paged pass and
// the prefix contraction, 1 runs paged_prefix_co_kernel where the plan marks
// it co-resident and paged_prefix_kernel elsewhere, 2 always
// paged_prefix_kernel, 0 two launches.
spkv_status run_decode(const spkv_batch *b, const spkv_kv *kv, const int32_t *cascade, float *out, float *lse,
                       void *ws, size_t ws_bytes, void *stream, const AppendIn *app = nullptr,
                       int single_launch = 1) {
    spkv_status st = spkv::validate_batch(b, kv);
    if (st != SPKV_OK) return st;
    if (!kv) return fail(SPKV_E_INVAL, "null kv");
    if (b->batch == 0) return SPKV_OK;
    if (!out) return fail(SPKV_E_INVAL, "null out");
    Plan p;
    st = spkv::make_plan(b, cascade, spkv::kPlanCUs, &p);
    if (st != SPKV_OK) return st;
    if (!ws || ws_bytes < (size_t)p.ws_bytes)
        return fail(SPKV_E_INVAL, "workspace too small: need " + std::to_string(p.ws_bytes) + " bytes");
    Args a = make_args(b, kv, p, ws);
    if (app) {
        a.append = 1;
        a.k_new = app->k_new;
        a.v_new = app->v_new;
    }
    // Streaming hint for the paged pass: only when it re-reads no HOT slab
    // (no member of a group that skips the prefix contraction).  A slab's
    // rows re-read by many requests' pieces are served by the caches, and
    // the non-temporal COLD reads slowed such steps down.
    a.cold_nt = 1;
    for (int r = 0; r < b->batch; ++r) {
        const int g = b->host_group_of[r];
        if (g >= 0 && g < b->num_groups && !((p.cascade.bits[g >> 5] >> (g & 31)) & 1u) && b->host_hot_len[g] > 0) {
            a.cold_nt = 0;
            break;
        }
    }
    hipStream_t hs = (hipStream_t)stream;
    const bool bf16 = b->dtype == SPKV_DTYPE_BF16;
    // The paged (HBM-bound) pass runs first, the prefix contraction (MFMA-
    // bound) second: the prefix pass's partial states are then still in the
    // last-level cache when the merge reads them, and their write-back does
    // not compete with the paged pass's reads.  Sub-batch i is entry i of
    // both paged passes.
    if (p.single_launch && single_launch != 0) {
        st = p.co_resident && single_launch == 1 ? launch_paged_prefix_co(a, p, app != nullptr, hs)
                                                 : launch_paged_prefix(a, p, app != nullptr, hs);
        if (st != SPKV_OK) return st;
    } else {
        for (size_t i = 0; i < p.flat.size(); ++i) {
            st = launch_flat(a, bf16, b->head_dim, p.flat[i], p.flat_head_groups, app ? app->slots : nullptr,
                             hs);
            if (st != SPKV_OK) return st;
        }
        if (p.run_prefix) {
            st = launch_prefix(a, p, b->head_dim, bf16, hs);
            if (st != SPKV_OK) return st;
        }
    }
    // Prefix partials per request (MFMA prefix pass): the split rule of the
    // prefix kernel applied to the host copies (validated by the plan).
    std::vector<uint8_t> prefix_np;
    if (a.prefix_mode == 1) {
        prefix_np.assign((size_t)b->batch, 0);
        for (int r = 0; r < b->batch; ++r) {
            const int g = b->host_group_of[r];
            if (g < 0 || g >= b->num_groups || !((p.cascade.bits[g >> 5] >> (g & 31)) & 1u)) continue;
            const int lp = b->host_hot_len[g];
            if (lp <= 0) continue;
            const int n = spkv::splits_for(lp, spkv::chunk_for(lp, a.prefix_tau, spkv::kPrefixSplitCap, a.prefix_granule));
            prefix_np[(size_t)r] = (uint8_t)std::min(n, spkv::kPrefixSplitCap);
        }
    }
    for (size_t i = 0; i < p.flat.size(); ++i) {
        st = launch_merge(a, b->head_dim, out, lse, p.flat[i], app ? app->slots : nullptr,
                          prefix_np.empty() ? nullptr : prefix_np.data(), hs);
        if (st != SPKV_OK) return st;
    }
    return SPKV_OK;
}

// ---------------------------------------------------------------------------
// Static scratch for spkv_decode_step_append_noalloc: the partial states of the
// split plan live in this file-scope device array instead of a caller
// workspace.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current.  Every call on one device shares the array.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = SPKV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) u32x4_t scratch[kScratchBytes / sizeof(u32x4_t)];

constexpr int kMaxDevices = 64;
struct ScratchTable {
    std::mutex mu;
    void *ptr[kMaxDevices] = {};
};
ScratchTable &scratch_table() {
    static ScratchTable t;
    return t;
}

spkv_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SPKV_E_HIP, std::string("noalloc: no current device: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SPKV_E_HIP, "noalloc: device index beyond the scratch table");
    ScratchTable &t = scratch_table();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPKV_E_HIP, std::string("noalloc: scratch address lookup failed: ") + hipGetErrorString(e));
        t.ptr[dev] = p;
    }
    *out = t.ptr[dev];
    return SPKV_OK;
}

spkv_status check_kv_shape(int32_t hkv, int32_t d, int32_t dtype) {
    if (hkv < 1 || hkv > spkv::kMaxKvHeads) return fail(SPKV_E_INVAL, "num_kv_heads must be 1..16");
    if (d != 64 && d != 128) return fail(SPKV_E_INVAL, "head_dim must be 64 or 128");
    if (dtype != SPKV_DTYPE_BF16 && dtype != SPKV_DTYPE_F32) return fail(SPKV_E_INVAL, "unknown dtype");
    return SPKV_OK;
}

}  // namespace

extern "C" {

spkv_status spkv_hot_write(const void *k_src, const void *v_src, int64_t base, int64_t lp, void *k_hot, void *v_hot,
                           int64_t hot_capacity, int32_t num_layers, int32_t layer, int32_t hkv, int32_t d,
                           int32_t dtype, void *stream) {
    spkv_status st = check_kv_shape(hkv, d, dtype);
    if (st != SPKV_OK) return st;
    if (base < 0 || lp < 0 || base + lp > hot_capacity) return fail(SPKV_E_INVAL, "hot_write: slab outside the pool");
    if (num_layers < 1 || layer < 0 || layer >= num_layers) return fail(SPKV_E_INVAL, "hot_write: layer outside the pool");
    if (lp == 0) return SPKV_OK;
    if (!k_src || !v_src || !k_hot || !v_hot) return fail(SPKV_E_INVAL, "hot_write: null pointer");
    const int esz = dtype == SPKV_DTYPE_BF16 ? 2 : 4;
    const int ppr = d * esz / 16;
    const int64_t total = lp * hkv * ppr;
    TimedLaunch tl(SPKV_KERNEL_CACHE, (hipStream_t)stream);
    tl.launch(hot_write_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (const u32x4_t *)k_src,
              (const u32x4_t *)v_src, (u32x4_t *)k_hot, (u32x4_t *)v_hot, base, lp, num_layers, layer, hkv, ppr);
    return check_launch("hot_write_kernel");
}

spkv_status spkv_reshape_and_cache(const void *k_new, const void *v_new, const int32_t *slot_mapping, int32_t n,
                                   void *k_cold, void *v_cold, int64_t cold_slots, int32_t hkv, int32_t d,
                                   int32_t dtype, void *stream) {
    spkv_status st = check_kv_shape(hkv, d, dtype);
    if (st != SPKV_OK) return st;
    if (n < 0 || cold_slots < 0) return fail(SPKV_E_INVAL, "reshape_and_cache: negative size");
    if (n == 0) return SPKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cold || !v_cold) return fail(SPKV_E_INVAL, "reshape_and_cache: null pointer");
    const int esz = dtype == SPKV_DTYPE_BF16 ? 2 : 4;
    const int pps = hkv * d * esz / 16;
    const int64_t total = (int64_t)n * pps;
    TimedLaunch tl(SPKV_KERNEL_CACHE, (hipStream_t)stream);
    tl.launch(reshape_and_cache_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (const u32x4_t *)k_new,
              (const u32x4_t *)v_new, slot_mapping, n, (u32x4_t *)k_cold, (u32x4_t *)v_cold, cold_slots, pps);
    return check_launch("reshape_and_cache_kernel");
}

spkv_status spkv_append_tokens(const void *k_new, const void *v_new, const int32_t *host_slots,
                               const int32_t *host_rows, int32_t n, void *k_cold, void *v_cold, int64_t cold_slots,
                               int32_t *tables, int32_t max_blocks, int32_t *lens, int32_t num_rows,
                               int32_t page_size, int32_t hkv, int32_t d, int32_t dtype, void *stream) {
    spkv_status st = check_kv_shape(hkv, d, dtype);
    if (st != SPKV_OK) return st;
    if (n < 0 || cold_slots < 0 || page_size < 1 || max_blocks < 0 || num_rows < 0)
        return fail(SPKV_E_INVAL, "append_tokens: bad size");
    if (n == 0) return SPKV_OK;
    if (!k_new || !v_new || !host_slots || !k_cold || !v_cold)
        return fail(SPKV_E_INVAL, "append_tokens: null pointer");
    if (tables && !lens) return fail(SPKV_E_INVAL, "append_tokens: tables without lens");
    for (int32_t i = 0; i < n; ++i) {
        if (host_slots[i] < 0 || host_slots[i] >= cold_slots)
            return fail(SPKV_E_INVAL, "append_tokens: slot " + std::to_string(host_slots[i]) + " of token " +
                                          std::to_string(i) + " outside the COLD pool");
        const int32_t r = host_rows ? host_rows[i] : i;
        if (tables && (r < 0 || r >= num_rows))
            return fail(SPKV_E_INVAL, "append_tokens: row " + std::to_string(r) + " of token " + std::to_string(i) +
                                          " outside [0, num_rows)");
    }
    const int esz = dtype == SPKV_DTYPE_BF16 ? 2 : 4;
    const int pps = hkv * d * esz / 16;
    for (int32_t i0 = 0; i0 < n; i0 += kAppendArgTokens) {
        AppendArgs aa;
        aa.n = std::min(kAppendArgTokens, n - i0);
        for (int i = 0; i < aa.n; ++i) {
            aa.slots[i] = host_slots[i0 + i];
            aa.rows[i] = host_rows ? host_rows[i0 + i] : i0 + i;
        }
        TimedLaunch tl(SPKV_KERNEL_CACHE, (hipStream_t)stream);
        const int64_t off = (int64_t)i0 * pps;
        tl.launch(append_tokens_kernel, dim3((unsigned)aa.n), dim3(128), 0, (const u32x4_t *)k_new + off,
                  (const u32x4_t *)v_new + off, aa, (u32x4_t *)k_cold, (u32x4_t *)v_cold, cold_slots, pps, tables,
                  max_blocks, lens, num_rows, page_size);
        st = check_launch("append_tokens_kernel");
        if (st != SPKV_OK) return st;
    }
    return SPKV_OK;
}

spkv_status spkv_copy_blocks(const int32_t *pairs, int32_t n, void *k_cold, void *v_cold, int32_t num_pages,
                             int32_t page_size, int32_t num_layers, int32_t hkv, int32_t d, int32_t dtype,
                             void *stream) {
    spkv_status st = check_kv_shape(hkv, d, dtype);
    if (st != SPKV_OK) return st;
    if (n < 0 || num_pages < 0 || page_size < 1) return fail(SPKV_E_INVAL, "copy_blocks: bad size");
    if (num_layers < 1 || num_layers > 65535) return fail(SPKV_E_INVAL, "copy_blocks: num_layers must be 1..65535");
    if (n == 0) return SPKV_OK;
    if (n > 65535) return fail(SPKV_E_INVAL, "copy_blocks: at most 65535 pairs per call");
    if (!pairs || !k_cold || !v_cold) return fail(SPKV_E_INVAL, "copy_blocks: null pointer");
    const int esz = dtype == SPKV_DTYPE_BF16 ? 2 : 4;
    const int64_t ppp = (int64_t)page_size * hkv * d * esz / 16;
    const unsigned gx = (unsigned)std::min<int64_t>(64, (ppp + 255) / 256);
    TimedLaunch tl(SPKV_KERNEL_CACHE, (hipStream_t)stream);
    tl.launch(copy_blocks_kernel, dim3(gx, (unsigned)n, (unsigned)num_layers), dim3(256), 0, pairs, (u32x4_t *)k_cold,
              (u32x4_t *)v_cold, num_pages, ppp);
    return check_launch("copy_blocks_kernel");
}

spkv_status spkv_block_table_append(int32_t *tables, int32_t max_blocks, int32_t *lens, int32_t num_rows,
                                    const int32_t *rows, const int32_t *slots, int32_t n, int32_t page_size,
                                    void *stream) {
    if (n < 0 || max_blocks < 0 || num_rows < 0 || page_size < 1) return fail(SPKV_E_INVAL, "block_table_append: bad size");
    if (n == 0) return SPKV_OK;
    if (!tables || !lens || !rows || !slots) return fail(SPKV_E_INVAL, "block_table_append: null pointer");
    TimedLaunch tl(SPKV_KERNEL_CACHE, (hipStream_t)stream);
    tl.launch(block_table_append_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, tables, max_blocks, lens,
              num_rows, rows, slots, n, page_size);
    return check_launch("block_table_append_kernel");
}

spkv_status spkv_cascade_decode(const spkv_batch *batch, const spkv_kv *kv, float *out, float *lse, void *ws,
                                size_t ws_bytes, void *stream) {
    return run_decode(batch, kv, nullptr, out, lse, ws, ws_bytes, stream);
}

spkv_status spkv_dense_decode(const spkv_batch *batch, const spkv_kv *kv, float *out, float *lse, void *ws,
                              size_t ws_bytes, void *stream) {
    spkv_status st = spkv::validate_batch(batch, kv);
    if (st != SPKV_OK) return st;
    std::vector<int32_t> none((size_t)std::max(1, batch->num_groups), 0);
    return run_decode(batch, kv, none.data(), out, lse, ws, ws_bytes, stream);
}

spkv_status spkv_decode_step(const spkv_batch *batch, const spkv_kv *kv, const spkv_dispatch_params *params,
                             float *out, float *lse, void *ws, size_t ws_bytes, void *stream, int32_t *cascade_out) {
    spkv_status st = spkv::validate_batch(batch, kv);
    if (st != SPKV_OK) return st;
    std::vector<int32_t> choice((size_t)std::max(1, batch->num_groups), 0);
    st = spkv_dispatch(batch, params, choice.data());
    if (st != SPKV_OK) return st;
    if (cascade_out)
        for (int g = 0; g < batch->num_groups; ++g) cascade_out[g] = choice[(size_t)g];
    return run_decode(batch, kv, choice.data(), out, lse, ws, ws_bytes, stream, nullptr,
                      params ? params->single_launch : 1);
}

spkv_status spkv_decode_step_append(const spkv_batch *batch, const spkv_kv *kv, const spkv_dispatch_params *params,
                                    const void *k_new, const void *v_new, const int32_t *host_slots, float *out,
                                    float *lse, void *ws, size_t ws_bytes, void *stream, int32_t *cascade_out) {
    spkv_status st = spkv::validate_batch(batch, kv);
    if (st != SPKV_OK) return st;
    if (!kv) return fail(SPKV_E_INVAL, "null kv");
    if (batch->dtype != SPKV_DTYPE_BF16) return fail(SPKV_E_INVAL, "decode_step_append: bf16 only");
    if (batch->batch > 0 && (!k_new || !v_new || !host_slots || !batch->host_cold_lens))
        return fail(SPKV_E_INVAL, "decode_step_append: null new-token argument");
    if (kv->cold_slots * (int64_t)batch->num_kv_heads >= ((int64_t)1 << 30))
        return fail(SPKV_E_INVAL, "decode_step_append: COLD pool too large (Hkv * cold_slots >= 2^30)");
    for (int i = 0; i < batch->batch; ++i) {
        const int64_t slot = host_slots[i];
        const int64_t len = batch->host_cold_lens[i];
        if (slot < 0 || slot >= kv->cold_slots)
            return fail(SPKV_E_INVAL, "decode_step_append: slot " + std::to_string(slot) + " of request " +
                                          std::to_string(i) + " outside the COLD pool");
        if (len < 1 || (len - 1) / batch->page_size >= batch->max_blocks)
            return fail(SPKV_E_INVAL, "decode_step_append: no block-table column for the new token of request " +
                                          std::to_string(i));
    }
    std::vector<int32_t> choice((size_t)std::max(1, batch->num_groups), 0);
    st = spkv_dispatch(batch, params, choice.data());
    if (st != SPKV_OK) return st;
    if (cascade_out)
        for (int g = 0; g < batch->num_groups; ++g) cascade_out[g] = choice[(size_t)g];
    const AppendIn app{k_new, v_new, host_slots};
    return run_decode(batch, kv, choice.data(), out, lse, ws, ws_bytes, stream, &app,
                      params ? params->single_launch : 1);
}

spkv_status spkv_decode_step_append_noalloc(const spkv_batch *batch, const spkv_kv *kv,
                                            const spkv_dispatch_params *params, const void *k_new,
                                            const void *v_new, const int32_t *host_slots, float *out, float *lse,
                                            void *stream, int32_t *cascade_out) {
    spkv_status st = spkv::validate_batch(batch, kv);
    if (st != SPKV_OK) return st;
    std::vector<int32_t> choice((size_t)std::max(1, batch->num_groups), 0);
    st = spkv_dispatch(batch, params, choice.data());
    if (st != SPKV_OK) return st;
    Plan p;
    st = spkv::make_plan(batch, choice.data(), spkv::kPlanCUs, &p);
    if (st != SPKV_OK) return st;
    if ((size_t)p.ws_bytes > kScratchBytes)
        return fail(SPKV_E_INVAL, "decode_step_append_noalloc: the plan needs " + std::to_string(p.ws_bytes) +
                                      " bytes of scratch, more than the static " +
                                      std::to_string(kScratchBytes) + " (use spkv_decode_step_append)");
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != SPKV_OK) return st;
    return spkv_decode_step_append(batch, kv, params, k_new, v_new, host_slots, out, lse, ws, kScratchBytes, stream,
                                   cascade_out);
}

}  // extern "C"

// A decode step recorded as a HIP graph and replayed with each step's kernel
// arguments: the step is captured on a private stream (capture enqueues no GPU
// work), the instantiated graph's nodes take the new arguments through
// hipGraphExecUpdate when the launches are the same as last time (same kernels
// and node count; grids may change), and the graph is re-instantiated
// otherwise.
struct spkv_graph {
    hipStream_t capture = nullptr;
    hipGraphExec_t exec = nullptr;
    int64_t instantiations = 0;
    int64_t updates = 0;
};

extern "C" {

spkv_status spkv_graph_create(spkv_graph **out) {
    if (!out) return fail(SPKV_E_INVAL, "graph_create: null out");
    auto *g = new spkv_graph();
    hipError_t e = hipStreamCreateWithFlags(&g->capture, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete g;
        return fail(SPKV_E_HIP, std::string("graph_create: stream: ") + hipGetErrorString(e));
    }
    *out = g;
    return SPKV_OK;
}

void spkv_graph_destroy(spkv_graph *g) {
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->capture) (void)hipStreamDestroy(g->capture);
    delete g;
}

spkv_status spkv_graph_decode_step_append(spkv_graph *g, const spkv_batch *batch, const spkv_kv *kv,
                                          const spkv_dispatch_params *params, const void *k_new, const void *v_new,
                                          const int32_t *host_slots, float *out, float *lse, void *ws,
                                          size_t ws_bytes, void *stream, int32_t *cascade_out,
                                          int32_t *instantiated_out) {
    if (!g) return fail(SPKV_E_INVAL, "graph_decode_step_append: null graph");
    if (instantiated_out) *instantiated_out = 0;
    // Argument errors come out of the capture as they would from the call itself.
    hipError_t e = hipStreamBeginCapture(g->capture, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) return fail(SPKV_E_HIP, std::string("graph: begin capture: ") + hipGetErrorString(e));
    spkv_status st = spkv_decode_step_append(batch, kv, params, k_new, v_new, host_slots, out, lse, ws, ws_bytes,
                                             g->capture, cascade_out);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(g->capture, &graph);
    if (st != SPKV_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (e != hipSuccess || !graph) return fail(SPKV_E_HIP, std::string("graph: end capture: ") + hipGetErrorString(e));
    bool updated = false;
    if (g->exec) {
        hipGraphExecUpdateResult res = hipGraphExecUpdateError;
        hipGraphNode_t bad = nullptr;
        updated = hipGraphExecUpdate(g->exec, graph, &bad, &res) == hipSuccess && res == hipGraphExecUpdateSuccess;
        (void)hipGetLastError();
        if (!updated) {
            (void)hipGraphExecDestroy(g->exec);
            g->exec = nullptr;
        }
    }
    if (!updated) {
        e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            (void)hipGraphDestroy(graph);
            g->exec = nullptr;
            return fail(SPKV_E_HIP, std::string("graph: instantiate: ") + hipGetErrorString(e));
        }
        g->instantiations += 1;
        if (instantiated_out) *instantiated_out = 1;
    } else {
        g->updates += 1;
    }
    (void)hipGraphDestroy(graph);
    e = hipGraphLaunch(g->exec, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SPKV_E_HIP, std::string("graph: launch: ") + hipGetErrorString(e));
    return SPKV_OK;
}

spkv_status spkv_merge_states(const float *o_a, const float *lse_a, const float *o_b, const float *lse_b, float *o,
                              float *lse, int64_t rows, int32_t head_dim, void *stream) {
    if (rows < 0 || head_dim <= 0) return fail(SPKV_E_INVAL, "merge_states: bad size");
    if (rows == 0) return SPKV_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o) return fail(SPKV_E_INVAL, "merge_states: null pointer");
    if (head_dim > 256 || 256 % head_dim) return fail(SPKV_E_INVAL, "merge_states: head_dim must divide 256");
    const int64_t total = rows * head_dim;
    TimedLaunch tl(SPKV_KERNEL_MERGE, (hipStream_t)stream);
    tl.launch(merge2_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, o_a, lse_a, o_b, lse_b, o, lse, rows,
              head_dim);
    return check_launch("merge2_kernel");
}

spkv_status spkv_timing_enable(int32_t on) {
    Timing &t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.on = on != 0;
    return SPKV_OK;
}

spkv_status spkv_timing_read(int32_t kernel, double *total_ms, int64_t *launches) {
    if (kernel < 0 || kernel >= SPKV_NUM_KERNELS || !total_ms || !launches)
        return fail(SPKV_E_INVAL, "timing_read: bad argument");
    Timing &t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    for (auto &r : t.pending) {
        if (hipEventSynchronize(r.b) != hipSuccess) return fail(SPKV_E_HIP, "timing_read: event wait failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(SPKV_E_HIP, "timing_read: elapsed time failed");
        t.total_ms[r.kernel] += ms;
        t.count[r.kernel] += 1;
        t.pool.push_back(r.a);
        t.pool.push_back(r.b);
    }
    t.pending.clear();
    *total_ms = t.total_ms[kernel];
    *launches = t.count[kernel];
    return SPKV_OK;
}

spkv_status spkv_timing_reset(void) {
    Timing &t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    for (auto &r : t.pending) {
        (void)hipEventSynchronize(r.b);
        t.pool.push_back(r.a);
        t.pool.push_back(r.b);
    }
    t.pending.clear();
    for (int k = 0; k < SPKV_NUM_KERNELS; ++k) {
        t.total_ms[k] = 0;
        t.count[k] = 0;
    }
    return SPKV_OK;
}

spkv_status spkv_device_cus(int32_t *cus_out) {
    if (!cus_out) return fail(SPKV_E_INVAL, "device_cus: null out");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPKV_E_HIP, "device_cus: no device");
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(SPKV_E_HIP, "device_cus: attribute query failed");
    *cus_out = n;
    return SPKV_OK;
}

}  // extern "C"
