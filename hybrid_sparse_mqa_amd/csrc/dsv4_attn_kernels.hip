// dsv4_attn_kernels.hip -- gfx950 kernels of the DeepSeek-V4 hybrid sparse MQA
// decode / verify path.
//
//  * gather_kernel: the paged gather stage alone (canonical slot lists).
//  * split kernels -- gather + KV tile load (+ FP8 decode) + scores + online
//    softmax + PV for one (query row, head block, key split); with a single
//    split they also apply the sink and write out / lse:
//      attn_ws_kernel<1>    bf16 KV, 32-head blocks with wave roles (two
//                           score waves, two PV waves one tile behind);
//      attn_wide_kernel<2>  bf16 KV, 64-head blocks (two head groups x two
//                           dim halves), one 32-key tile per step;
//      attn_wide_kernel<1>  bf16 KV, 32-head blocks (four dim quarters),
//                           fewer splits for the same parallelism;
//      attn_narrow_kernel   bf16 KV, 16-head blocks, four independent waves;
//      attn_fp8_kernel      packed FP8 KV, 64-head blocks.
//  * merge_kernel: log-sum-exp merge of the split partials with the per-head
//    sink folded in once (test-matrix page, attention-sink correction).
//    All query heads share each KV row (MQA with one KV head, walk-through
//    page section 1), so a key tile is fetched from HBM once per workgroup into
//    LDS and feeds both products on bf16 MFMA:
//        S^T[keys, heads]  = K[keys, d] . Q^T[d, heads]
//        O^T[d, heads]    += K^T[d, keys] . P^T[keys, heads]      (V = K)
//    The second product reduces over keys.  The bf16 kernels stream key rows
//    straight from HBM into LDS (global_load_lds) and read PV operands with
//    the gfx950 transposing LDS read (ds_read_b64_tr_b16).  The FP8 kernel
//    streams the raw records into LDS the same way and converts the codes
//    into bf16 operands in registers: row-wise reads for S, the 8-bit
//    transposing read (ds_read_b64_tr_b8) for PV.
//
// Work items (row, head block, split) are laid out so that consecutive
// items -- the head blocks and splits of one row -- go to the same XCD
// (workgroups are dispatched to the 8 XCDs round robin), which keeps a row's
// Q and key rows shared in one L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "dsv4_launch.h"

namespace dsv4 {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Two OCP E4M3FN codes (bytes 0, 1 of w, or bytes 2, 3 with kHi) -> two
// bf16 in one word, the first code in the low half: the gfx950 conversion
// instruction with scale 1.  Every E4M3 value, subnormals included, is exact
// in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}


// vmcnt-only wait (expcnt / lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Direct global -> LDS copy of 16 bytes per lane, with a byte offset OFF
// folded into the instruction (a 13-bit signed immediate): lane i's bytes
// from src + OFF land at LDS byte address lds_row + 16*i.  The instruction
// adds the offset to the LDS address as well as to the global one, so M0
// (the wave-uniform LDS base) is set to the destination minus the offset.
// Issued as inline asm so that the compiler does not treat every later LDS
// access as dependent on it; callers wait with wait_vmcnt() and a barrier.
// M0 is saved and restored around the copy, with the one wait state the
// hardware needs between an M0 write and an LDS-DMA instruction.
template <int OFF>
__device__ __forceinline__ void dma16_off(const void* src, uint32_t lds_row) {
    static_assert(OFF >= 0 && OFF < 4096, "global offset is 13-bit signed");
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_row - OFF);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:%3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base), "n"(OFF)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void*)p;
}

struct Item {
    int t, hb, s;
};

// Work item of this workgroup (XCD-aware: consecutive items -- the splits of
// one row -- share an XCD, since workgroups go to the 8 XCDs round robin).
// Returns false for a spare workgroup of the rounded-up grid, whose item is
// clamped into range so that it can issue its first loads like the others
// before leaving (no branch splits the kernel-argument loads).
__device__ __forceinline__ bool decode_item(const AttnArgs& a, Item& it) {
    const int per_xcd = (a.n_items + 7) >> 3;
    const int slot_in_xcd = blockIdx.x >> 3;
    const int raw = (blockIdx.x & 7) * per_xcd + slot_in_xcd;
    const bool live = slot_in_xcd < per_xcd && raw < a.n_items;
    const int item = min(raw, a.n_items - 1);
    it.s = item % a.splits;
    const int th = item / a.splits;
    it.hb = th % a.head_blocks;
    it.t = th / a.head_blocks;
    return live;
}

// Recording builds (the test hook): work-item index of the key records.
__device__ __forceinline__ int64_t dbg_unit(const AttnArgs& a, const Item& it) {
    return ((int64_t)it.t * a.head_blocks + it.hb) * a.splits + it.s;
}

// The kernel arguments that the first round of loads depends on, made
// available at one point so that they arrive in one round of scalar loads
// (left to itself the compiler fetches them in several dependent rounds, each
// a memory round trip before the loads that need it can go out).
__device__ __forceinline__ void fetch_args(const AttnArgs& a) {
    asm volatile("" ::"s"(a.m.seq_lens), "s"(a.m.qo_indptr), "s"(a.m.c4), "s"(a.m.c4_ld), "s"(a.m.ext_table),
                 "s"(a.m.ext_ld), "s"(a.m.swa_table), "s"(a.m.swa_ld), "s"(a.m.K), "s"(a.m.B), "s"(a.m.R),
                 "s"(a.m.W), "s"(a.q), "s"(a.q_s0), "s"(a.q_s1), "s"(a.T), "s"(a.H), "s"(a.chunk), "s"(a.splits),
                 "s"(a.head_blocks), "s"(a.n_items), "s"(a.ext_pages), "s"(a.zero_row));
}

// Slot list of keys [k0, k0 + n_here) of row t into s_slot.  One round of
// loads fetches the request's extra page-table row (cached in LDS) and, per
// key, its window page entry or its C4 index; every address is clamped into
// range so that no load sits under a per-lane branch and all of them are in
// flight together.  Compressed slots then resolve through the LDS table (or,
// for a table longer than kTableCap pages, through one more round of loads).
template <int kMaxKeys = kMaxSplitKeys>
__device__ __forceinline__ void build_slots(const AttnArgs& a, const RowKeys& rk, int t, int k0, int n_here,
                                            int32_t* s_slot, int32_t* s_table, int tid) {
    constexpr int kU = kMaxKeys / 256;
    constexpr int kTU = kTableCap / 256;
    const bool cached_table = a.m.R != 0 && a.ext_pages <= kTableCap;
    const int32_t* ext_row = a.m.ext_table + (int64_t)rk.r * a.m.ext_ld;
    const int32_t* swa_row = a.m.swa_table + (int64_t)rk.r * a.m.swa_ld;
    const int32_t* c4_row = a.m.R == 4 ? a.m.c4 + (int64_t)t * a.m.c4_ld : swa_row;
    int32_t tab[kTU];
    if (cached_table) {
#pragma unroll
        for (int j = 0; j < kTU; ++j) tab[j] = ext_row[min(tid + 256 * j, a.ext_pages - 1)];
    }
    // Raw loads first (all kU of them, clamped), arithmetic after, so that no
    // wait for one load comes before the next load is issued.
    int32_t raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int e = k0 + tid + 256 * u;
        const int x = rk.swa_lo + min(e, rk.n_swa - 1);
        const int c = min(max(e - rk.n_swa, 0), max(a.m.K - 1, 0));
        raw[u] = *((e < rk.n_swa || a.m.R != 4) ? swa_row + (x >> 8) : c4_row + c);  // K >= 1 when R == 4
    }
    int32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int e = k0 + tid + 256 * u;
        const int x = rk.swa_lo + min(e, rk.n_swa - 1);
        v[u] = e < rk.n_swa ? raw[u] * kPage + (x & (kPage - 1)) : (a.m.R == 4 ? raw[u] : e - rk.n_swa);
    }
#pragma unroll
    for (int j = 0; j < kTU; ++j)
        if (cached_table && tid + 256 * j < a.ext_pages) s_table[tid + 256 * j] = tab[j];
    __syncthreads();  // s_table ready
    // A table too long for LDS: one more round of (clamped) loads.
    int32_t pg[kU] = {};
    if (a.m.R != 0 && !cached_table) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const bool ext = k0 + tid + 256 * u >= rk.n_swa && v[u] >= 0;
            pg[u] = ext_row[ext ? min(v[u] >> 8, a.ext_pages - 1) : 0];
        }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int i = tid + 256 * u;
        if (i < n_here) {
            int32_t slot = v[u];
            if (k0 + i >= rk.n_swa && slot >= 0)
                slot = (cached_table ? s_table[slot >> 8] : pg[u]) * kPage + (slot & (kPage - 1));
            s_slot[i] = slot;
        }
    }
    __syncthreads();  // slot list ready
}

// Slot list of keys [k0, k0 + n_here) of row t in compressed-first order
// (list index i < n_ext: compressed entry i, C4 entries as listed with -1
// for unused ones; i >= n_ext: window position swa_lo + (i - n_ext)), in two
// steps.  prefetch_slots issues the loads that need nothing from the row's
// request bounds -- the C4 indices of the split's keys and the extra
// page-table row of the request guessed from the row index (t B / T, exact
// when every request has equally many query rows) -- so that they are in
// flight with the bounds; finish_slots reloads the table row on a wrong
// guess, fetches the window keys' page entries (which need the row's
// position), and writes s_slot.  Every load is unconditional, from a
// clamped index or from the zero row.
struct SlotPrefetch {
    int32_t raw[kMaxSplitKeys / 256];  // C4 index of key k0 + tid + 256 u
    int32_t tab[kTableCap / 256];      // extra page-table entries tid + 256 j of the guessed request
    int r_guess;
};

__device__ __forceinline__ void prefetch_slots(const AttnArgs& a, int t, int k0, int tid, SlotPrefetch& pf) {
    constexpr int kU = kMaxSplitKeys / 256, kTU = kTableCap / 256;
    pf.r_guess = min(a.m.B - 1, (int)((int64_t)t * a.m.B / max(a.T, 1)));
    const int32_t* zero = (const int32_t*)a.zero_row;
    const bool cached = a.m.R != 0 && a.ext_pages <= kTableCap;
    const int32_t* ext_row = cached ? a.m.ext_table + (int64_t)pf.r_guess * a.m.ext_ld : zero;
#pragma unroll
    for (int j = 0; j < kTU; ++j) pf.tab[j] = ext_row[cached ? min(tid + 256 * j, a.ext_pages - 1) : 0];
    const bool c4 = a.m.R == 4;
    const int32_t* c4_row = c4 ? a.m.c4 + (int64_t)t * a.m.c4_ld : zero;
#pragma unroll
    for (int u = 0; u < kU; ++u) pf.raw[u] = c4_row[c4 ? min(k0 + tid + 256 * u, max(a.m.K - 1, 0)) : 0];
}

__device__ __forceinline__ void finish_slots(const AttnArgs& a, const RowKeys& rk, int k0, int n_here,
                                             SlotPrefetch& pf, int32_t* s_slot, int32_t* s_table, int tid) {
    constexpr int kU = kMaxSplitKeys / 256, kTU = kTableCap / 256;
    const bool cached = a.m.R != 0 && a.ext_pages <= kTableCap;
    const int32_t* ext_row = a.m.ext_table + (int64_t)rk.r * a.m.ext_ld;
    if (cached && rk.r != pf.r_guess) {  // a wrong guess: the row's own table
#pragma unroll
        for (int j = 0; j < kTU; ++j) pf.tab[j] = ext_row[min(tid + 256 * j, a.ext_pages - 1)];
    }
    // Page entries of this thread's window keys (clamped for the others).
    const int32_t* swa_row = a.m.swa_table + (int64_t)rk.r * a.m.swa_ld;
    int32_t wpg[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int w = min(max(k0 + tid + 256 * u - rk.n_ext, 0), rk.n_swa - 1);
        wpg[u] = swa_row[(rk.swa_lo + w) >> 8];
    }
#pragma unroll
    for (int j = 0; j < kTU; ++j)
        if (cached && tid + 256 * j < a.ext_pages) s_table[tid + 256 * j] = pf.tab[j];
    __syncthreads();  // s_table ready
    // A table too long for LDS: one more round of (clamped) loads.
    int32_t pg[kU] = {};
    if (a.m.R != 0 && !cached) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int e = k0 + tid + 256 * u;
            const int c = a.m.R == 4 ? pf.raw[u] : e;
            pg[u] = ext_row[e < rk.n_ext && c >= 0 ? min(c >> 8, a.ext_pages - 1) : 0];
        }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int i = tid + 256 * u;
        if (i < n_here) {
            const int e = k0 + i;
            int32_t slot;
            if (e < rk.n_ext) {
                const int c = a.m.R == 4 ? pf.raw[u] : e;
                slot = c < 0 ? -1 : (cached ? s_table[c >> 8] : pg[u]) * kPage + (c & (kPage - 1));
            } else {
                slot = wpg[u] * kPage + ((rk.swa_lo + e - rk.n_ext) & (kPage - 1));
            }
            s_slot[i] = slot;
        }
    }
    __syncthreads();  // slot list ready
}

// ---- Compressed-first key lists (the wide kernels) -------------------------
// The wide kernels walk a row's keys compressed entries first: list index
// i < n_ext is compressed entry i (C4: c4_indices[t][i], negative = unused;
// C128: entry i), and i >= n_ext is window position swa_lo + (i - n_ext).
// (The softmax does not depend on the order; the canonical order of the
// gather entry point is unchanged.)
//
// Each lane resolves only the keys whose row addresses it holds: the rows
// it copies itself for tiles 0..2, and one row of every later tile, which
// it hands to the copying lane through a cross-lane permute (see
// lane_key).  The C4 indices of a split depend only on the query row, and
// the extra page-table row only on the request, so both are requested in the
// first round of loads, together with the request bounds, for the request a
// row has when every request has equally many query rows (t * B / T); a
// wrong guess costs one reload.  C128 entries need no index: the lane loads
// the page-table entry of each of its keys' pages directly.  Window slots
// need the row's position, so they come from a second round: one or a few
// page-table entries at uniform addresses, read with scalar loads, which a
// wave can wait for without waiting for tile copies already in flight.
constexpr int kAdRegs = kMaxSplitKeys / 256;  // permuted row addresses per lane
constexpr int kLaneKeys = kAdRegs + 3;

// Split-relative key of lane key q of lane l in wave w: q < kAdRegs is row
// 8w + (l & 7) of tile 8q + (l >> 3); q = kAdRegs + j is the row lane l
// copies in tile j (row 8w + ((l >> 1) & 7)).
__device__ __forceinline__ int lane_key(int q, int w, int l) {
    return q < kAdRegs ? 256 * q + 32 * (l >> 3) + 8 * w + (l & 7) : 32 * (q - kAdRegs) + 8 * w + ((l >> 1) & 7);
}

struct ExtPrefetch {
    int32_t e[kLaneKeys];          // C4: index of each lane key's entry; C128: page-table entry of its page
    int32_t tab[kTableCap / 256];  // C4: extra page-table entries tid + 256*j
    int r_guess;                   // the request the page-table loads assume
};

// Every load is unconditional (from the zero row where the ratio does not
// need it), so that no branch splits them.
__device__ __forceinline__ void prefetch_ext(const AttnArgs& a, int t, int k0, int w, int l, int tid, ExtPrefetch& pf) {
    pf.r_guess = min(a.m.B - 1, (int)((int64_t)t * a.m.B / max(a.T, 1)));
    const bool c4 = a.m.R == 4, c128 = a.m.R == 128;
    const bool table = c4 && a.ext_pages <= kTableCap;
    const int32_t* zero = (const int32_t*)a.zero_row;
    const int32_t* ext_row = c4 || c128 ? a.m.ext_table + (int64_t)pf.r_guess * a.m.ext_ld : zero;
    const int32_t* c4_row = c4 ? a.m.c4 + (int64_t)t * a.m.c4_ld : zero;
#pragma unroll
    for (int q = 0; q < kLaneKeys; ++q) {
        const int key = k0 + lane_key(q, w, l);
        const int32_t* src = c4 ? c4_row + min(key, a.m.K - 1) : ext_row + (c128 ? min(key >> 8, a.ext_pages - 1) : 0);
        pf.e[q] = *src;
    }
    const int32_t* tab_row = table ? ext_row : zero;
#pragma unroll
    for (int j = 0; j < kTableCap / 256; ++j) {
        const int32_t* src = tab_row + (table ? min(tid + 256 * j, a.ext_pages - 1) : 0);
        pf.tab[j] = *src;
    }
}

// Row address of every lane key that is a compressed entry of the split; the
// zero row for unused C4 entries, keys past the split and window keys (which
// the caller fills in later).  Bit q of valid (q < kAdRegs): the key is used.
__device__ __forceinline__ void ext_addresses(const AttnArgs& a, const RowKeys& rk, int k0, int n_here, int w,
                                              int l, int tid, ExtPrefetch& pf, int32_t* s_table,
                                              uint64_t (&addr)[kLaneKeys], uint32_t& valid) {
    const int32_t* ext_row = a.m.ext_table + (int64_t)rk.r * a.m.ext_ld;
    int32_t slot[kLaneKeys];
    valid = 0;
    if (a.m.R == 128) {
        if (rk.r != pf.r_guess) {  // uniform: the guessed request was wrong
#pragma unroll
            for (int q = 0; q < kLaneKeys; ++q) pf.e[q] = ext_row[min((k0 + lane_key(q, w, l)) >> 8, a.ext_pages - 1)];
            // Wait here, on this path only: otherwise the compiler waits for
            // every later load (Q) below, on the common path too.
            wait_vmcnt<0>();
        }
#pragma unroll
        for (int q = 0; q < kLaneKeys; ++q) slot[q] = pf.e[q] * kPage + ((k0 + lane_key(q, w, l)) & (kPage - 1));
    } else if (a.m.R == 4) {
        if (a.ext_pages <= kTableCap) {  // uniform: the request's table goes through LDS
            if (rk.r != pf.r_guess) {
#pragma unroll
                for (int j = 0; j < kTableCap / 256; ++j) pf.tab[j] = ext_row[min(tid + 256 * j, a.ext_pages - 1)];
                wait_vmcnt<0>();  // on this path only (see above)
            }
#pragma unroll
            for (int j = 0; j < kTableCap / 256; ++j)
                if (tid + 256 * j < a.ext_pages) s_table[tid + 256 * j] = pf.tab[j];
            __syncthreads();  // s_table ready
            int32_t pg[kLaneKeys];  // read unconditionally (clamped), so that the reads go out together
#pragma unroll
            for (int q = 0; q < kLaneKeys; ++q) pg[q] = s_table[pf.e[q] >= 0 ? min(pf.e[q] >> 8, a.ext_pages - 1) : 0];
#pragma unroll
            for (int q = 0; q < kLaneKeys; ++q) slot[q] = pf.e[q] < 0 ? -1 : pg[q] * kPage + (pf.e[q] & (kPage - 1));
        } else {  // a table too long for LDS: one more round of (clamped) loads
            int32_t pg[kLaneKeys];
#pragma unroll
            for (int q = 0; q < kLaneKeys; ++q) pg[q] = ext_row[pf.e[q] >= 0 ? min(pf.e[q] >> 8, a.ext_pages - 1) : 0];
            wait_vmcnt<0>();  // on this path only (see above)
#pragma unroll
            for (int q = 0; q < kLaneKeys; ++q) slot[q] = pf.e[q] < 0 ? -1 : pg[q] * kPage + (pf.e[q] & (kPage - 1));
        }
    } else {
#pragma unroll
        for (int q = 0; q < kLaneKeys; ++q) slot[q] = -1;
    }
#pragma unroll
    for (int q = 0; q < kLaneKeys; ++q) {
        const int key = lane_key(q, w, l);
        const bool ext = key < n_here && k0 + key < rk.n_ext;
        addr[q] = ext && slot[q] >= 0 ? (uint64_t)(uintptr_t)(a.ext_pool + (int64_t)slot[q] * a.ext_row_bytes)
                                      : (uint64_t)(uintptr_t)a.zero_row;
        if (q < kAdRegs && key < n_here && (!ext || slot[q] >= 0)) valid |= 1u << q;  // window keys are always used
    }
}

// Page-table entries of the window pages a split touches: pages pg_lo ..
// pg_lo + 4 (clamped to the last page touched), which covers any split of at
// most 1024 window keys.  They are issued as uniform scalar loads whose
// results the compiler is not told about: wait_swa_pages() must run before
// any use, and no LDS access may come in between (scalar and LDS loads share
// a counter, and a partial LDS wait could pass while a scalar load is still
// pending).
struct SwaPages {
    int32_t e[5];
    int pg_lo;
    bool any;  // the split holds window keys
};

__device__ __forceinline__ SwaPages issue_swa_pages(const AttnArgs& a, const RowKeys& rk, int k0, int n_here) {
    SwaPages sp;
    const int i_lo = max(k0, rk.n_ext), i_hi = min(k0 + n_here, rk.n_ext + rk.n_swa);
    sp.any = __builtin_amdgcn_readfirstlane(i_lo < i_hi ? 1 : 0) != 0;  // uniform: rk is
    sp.pg_lo = __builtin_amdgcn_readfirstlane((rk.swa_lo + max(i_lo - rk.n_ext, 0)) >> 8);
    const int pg_hi = __builtin_amdgcn_readfirstlane(sp.any ? (rk.swa_lo + (i_hi - 1 - rk.n_ext)) >> 8 : sp.pg_lo);
    const int32_t* row = a.m.swa_table + (int64_t)__builtin_amdgcn_readfirstlane(rk.r) * a.m.swa_ld;
#pragma unroll
    for (int k = 0; k < 5; ++k) sp.e[k] = 0;
    if (sp.any) {  // only then are pg_lo .. pg_hi pages of the row
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int32_t* p = row + min(sp.pg_lo + k, pg_hi);
            asm volatile("s_load_dword %0, %1, 0x0" : "=s"(sp.e[k]) : "s"(p) : "memory");
        }
    }
    return sp;
}

__device__ __forceinline__ void wait_swa_pages(SwaPages& sp) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(sp.e[0]), "+s"(sp.e[1]), "+s"(sp.e[2]), "+s"(sp.e[3]), "+s"(sp.e[4])
                 :
                 : "memory");
}

// Sum the S^T partials of the two waves that share a head half (they cover
// the two dim halves).  Layout [wave][chunk][lane] in 16-byte units keeps the
// 16-byte accesses of consecutive lanes contiguous (no bank conflicts).
__device__ __forceinline__ void exchange_partial(float* s_sx, int w, int l, f32x16& sacc) {
    f32x4* mine = (f32x4*)s_sx + w * 256 + l;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
    __syncthreads();
    const f32x4* other = (const f32x4*)s_sx + (w ^ 1) * 256 + l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 o = other[64 * q];
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[4 * q + j] += o[j];
    }
}

// The same over the four waves that share all 32 heads (each holding one
// dim quarter), added pairwise -- (own + w^1) + (w^2 + w^3) -- so that every
// wave gets the same sums (each addition is commutative).
__device__ __forceinline__ void exchange_partial4(float* s_sx, int w, int l, f32x16& sacc) {
    f32x4* mine = (f32x4*)s_sx + w * 256 + l;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
    __syncthreads();
    f32x4 o[3][4];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
        const f32x4* other = (const f32x4*)s_sx + (w ^ v) * 256 + l;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[v - 1][q] = other[64 * q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[4 * q + j] = (sacc[4 * q + j] + o[0][q][j]) + (o[1][q][j] + o[2][q][j]);
}

// Multiply every output accumulator by alpha in place.  Each register is
// read out of the accumulation file, scaled and written back by one short
// asm sequence, so the accumulators never have to live in VGPRs (letting the
// compiler do it makes the register allocator spill the whole tile).
// Wait states: one between the read-out and its VALU use, and a few before
// any later MFMA reads the rewritten registers.
template <int NB>
__device__ __forceinline__ void scale_accumulators(f32x16 (&oacc)[NB], float alpha) {
    // Enough wait states for the last MFMA that wrote an accumulator to
    // retire before the first read-out.
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3");
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float x = oacc[mb][e];
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "s_nop 1\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            oacc[mb][e] = x;
        }
    asm volatile("s_nop 4");
}

// The same for 16x16 accumulator tiles (four registers each).
template <int NB>
__device__ __forceinline__ void scale_accumulators(f32x4 (&oacc)[NB], float alpha) {
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3");
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = oacc[mb][e];
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "s_nop 1\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            oacc[mb][e] = x;
        }
    asm volatile("s_nop 4");
}

// Online-softmax step for one 32-key tile (base 2).  `sacc` holds this
// wave's S^T accumulators already summed over all 512 dims: register r is
// head (l & 31), tile key 8*(r >> 2) + 4*(l >> 5) + (r & 3), so lanes l and
// l ^ 32 hold the two halves of a head's keys.  Produces the bf16 P^T
// operands of the two PV k-steps.  The running reference m_run only moves
// when a score exceeds it by more than 2^8 (probabilities stay <= 256), so
// the output accumulators are rescaled on a tiny fraction of tiles, and only
// then do the two lanes of a head agree on a new reference (one cross-lane
// exchange).  l_run is this lane's share of the denominator (its 16 keys per
// tile); the two shares are added once, in write_result.  A tile whose 32
// keys are all valid skips the masking.
template <bool kFp8, int NB>
__device__ __forceinline__ void softmax_tile(const f32x16& s_all, uint64_t vmask, float scale_log2, int l,
                                             const float (&sc_key)[16], float& m_run, float& l_run,
                                             f32x16 (&oacc)[NB], bf16x8 (&pb)[2], bf16x8 (&pbs)[2]) {
    float sv[16];
    float tmax = -INFINITY;
    if ((uint32_t)vmask == 0xFFFFFFFFu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sv[r] = s_all[r] * scale_log2;
            tmax = fmaxf(tmax, sv[r]);
        }
    } else {
        const uint32_t mine = (uint32_t)(vmask >> (4 * (l >> 5)));  // bit 8q + j: key 8q + 4*(l >> 5) + j
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int bit = 8 * (r >> 2) + (r & 3);
            const float x = s_all[r] * scale_log2;
            sv[r] = ((mine >> bit) & 1u) ? x : -INFINITY;
            tmax = fmaxf(tmax, sv[r]);
        }
    }
    if (__any(tmax > m_run + kRescaleLog2)) {
        const float hmax = fmaxf(tmax, __shfl_xor(tmax, 32));  // the head's tile maximum
        const bool grow = hmax > m_run + kRescaleLog2;
        const float m_target = grow ? hmax : m_run;
        const float alpha = fast_exp2(m_run - m_target);  // 0 while nothing was accumulated
        if (__any(grow && m_run != -INFINITY)) {
            scale_accumulators(oacc, alpha);
        }
        l_run *= alpha;
        m_run = m_target;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(sv[r] - m_use);
        psum += pr;
        pb[r >> 3][r & 7] = (__bf16)pr;
        if constexpr (kFp8) pbs[r >> 3][r & 7] = (__bf16)(pr * sc_key[r]);
    }
    l_run += psum;
}

// Epilogue of the wide layouts.  kHH head groups of 32 heads; wave (hh, dq)
// holds O^T for heads 32*hh + (l & 31) and its slice of kDims = 128*kHH dims:
// accumulator r of tile mb is dim kDims*dq + 32*mb + 8*(r >> 2) + 4*(l >> 5) +
// (r & 3).  One split: apply the sink and write out / lse.  Several: publish
// the normalised partial (in bf16: it is a convex combination of key rows,
// so 8 significant bits keep it within the output's own rounding; an empty
// split publishes zeros) and its base-2 log-sum-exp (-inf for an empty
// split) for merge_kernel.  The bf16 rows are first assembled in LDS
// (stage_lo / stage_hi for the head groups: 32 head rows of 1 KiB, 16-byte
// chunk c of row r at chunk c ^ r), so that every global store instruction
// writes one whole 1 KiB row.  The caller's LDS must be free: the first
// barrier below waits until every wave is done with it.
template <int kHH>
__device__ __forceinline__ void write_result(const AttnArgs& a, const Item& it, int hh, int dq, int l,
                                             const f32x16 (&oacc)[4 * kHH], float m_run, float l_half,
                                             uint8_t* stage_lo, uint8_t* stage_hi) {
    constexpr int kGroup = 4 / kHH;
    constexpr int kRows = 32 / kGroup;  // head rows stored by each wave
    uint8_t* stage = hh ? stage_hi : stage_lo;
    const float l_run = l_half + __shfl_xor(l_half, 32);  // both halves of the head's keys
    const int my_head = it.hb * 32 * kHH + hh * 32 + (l & 31);
    const bool head_ok = my_head < a.H;
    float f = 0.f, lse2 = -INFINITY;
    if (a.splits == 1) {
        const float sig = a.sink != nullptr && head_ok ? a.sink[my_head] * kLog2e : -INFINITY;
        const float M = fmaxf(m_run, sig);
        if (M != -INFINITY) {
            const float em = fast_exp2(m_run - M);
            const float den = l_run * em + fast_exp2(sig - M);
            f = em / den;
            lse2 = M + fast_log2(den);
        }
    } else if (l_run > 0.f) {
        f = 1.f / l_run;
        lse2 = m_run + fast_log2(l_run);
    }
    __syncthreads();  // every wave is done with the LDS the rows are staged in
    {
        const int r = l & 31;
        uint8_t* base = stage + r * 1024 + 8 * (l >> 5);
#pragma unroll
        for (int mb = 0; mb < 4 * kHH; ++mb) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int c = dq * 16 * kHH + 4 * mb + qd;
                const f32x16& o = oacc[mb];
                *(u32x2*)(base + 16 * (c ^ r)) = u32x2{pack_bf16x2(o[4 * qd] * f, o[4 * qd + 1] * f),
                                                       pack_bf16x2(o[4 * qd + 2] * f, o[4 * qd + 3] * f)};
            }
        }
    }
    __syncthreads();
    // Wave (hh, dq) stores rows kRows*dq .. +kRows of its head group; lane l
    // moves the row's 16-byte chunk l.  All LDS reads go out first, then the
    // stores (rows of heads past H are skipped), so that no store waits for
    // the next read.
    u32x4 v[kRows];
#pragma unroll
    for (int e = 0; e < kRows; ++e) {
        const int r = kRows * dq + e;
        v[e] = *(const u32x4*)(stage + r * 1024 + 16 * (l ^ r));
    }
    const int head0 = it.hb * 32 * kHH + hh * 32 + kRows * dq;
    const int n_rows = min(kRows, a.H - head0);  // uniform
    // Streaming stores: nothing in this kernel reads these rows again.
    if (a.splits == 1) {
        uint16_t* orow = a.out + (int64_t)it.t * a.out_s0 + (int64_t)head0 * a.out_s1 + 8 * l;
#pragma unroll
        for (int e = 0; e < kRows; ++e) {
            if (e < n_rows) {
                __builtin_nontemporal_store(u32x2{v[e][0], v[e][1]}, (u32x2*)(orow + e * a.out_s1));  // 8-byte aligned rows
                __builtin_nontemporal_store(u32x2{v[e][2], v[e][3]}, (u32x2*)(orow + e * a.out_s1 + 4));
            }
        }
    } else {
        uint16_t* prow = a.ws_o + (((int64_t)it.t * a.splits + it.s) * a.H + head0) * kHeadDim + 8 * l;
#pragma unroll
        for (int e = 0; e < kRows; ++e)
            if (e < n_rows) __builtin_nontemporal_store(v[e], (u32x4*)(prow + e * kHeadDim));
    }
    if (head_ok && dq == 0 && l < 32) {
        if (a.splits == 1) {
            if (a.lse != nullptr) a.lse[(int64_t)it.t * a.lse_s0 + my_head] = lse2 * kLn2;
        } else {
            a.ws_lse[((int64_t)it.t * a.splits + it.s) * a.H + my_head] = lse2;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Gather stage on its own: one workgroup per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs g) {
    __shared__ int wave_count[4];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const RowKeys rk = row_keys(g.m, t, tid & 63);
    int32_t* out = g.slots + (int64_t)t * g.slots_ld;
    for (int i = tid; i < rk.n_swa; i += 256) out[i] = list_slot(g.m, rk, t, i);
    int n_ext = 0;
    if (g.m.R == 128) {
        for (int e = tid; e < rk.n_ext; e += 256) out[rk.n_swa + e] = list_slot(g.m, rk, t, rk.n_swa + e);
        n_ext = rk.n_ext;
    } else if (g.m.R == 4) {
        // Stream compaction of the used C4 entries, keeping list order.
        const int lane = tid & 63, w = tid >> 6;
        for (int base = 0; base < rk.n_ext; base += 256) {
            const int e = base + tid;
            int32_t slot = -1;
            if (e < rk.n_ext) slot = list_slot(g.m, rk, t, rk.n_swa + e);
            const bool used = slot >= 0;
            const uint64_t ball = __ballot(used);
            const int before = __popcll(ball & ((1ull << lane) - 1ull));
            if (lane == 0) wave_count[w] = __popcll(ball);
            __syncthreads();
            int off = n_ext;
            for (int j = 0; j < w; ++j) off += wave_count[j];
            if (used) out[rk.n_swa + off + before] = slot;
            const int total = wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
            __syncthreads();
            n_ext += total;
        }
    }
    for (int i = rk.n_swa + n_ext + tid; i < g.slots_ld; i += 256) out[i] = -1;
    if (tid == 0) {
        g.counts[2 * t] = rk.n_swa;
        g.counts[2 * t + 1] = n_ext;
    }
}

// ---------------------------------------------------------------------------
// bf16 KV, wide layouts: one workgroup per (row, block of 32*kHH heads, key
// split).  kHH = 2: wave w = 2*hh + dq owns heads [32*hh, 32*hh + 32) and
// head dims [256*dq, 256*dq + 256) of every tile; kHH = 1: wave w = dq owns
// head dims [128*dq, 128*dq + 128) of all 32 heads.  The waves of one head
// group (2 or 4) each reduce the scores over their dims and sum the partials
// through LDS, in wave order, so that all of them hold the same scores and
// run the same softmax.  Key rows stream from HBM into a 4-stage LDS ring
// with direct global->LDS loads (no VGPR staging).
//
// Tile layout in LDS (32 KiB per stage).  Rows 8g .. 8g+7 form group g; the
// 512 bytes of dim half dh of those rows form four 1 KiB blocks m (128-byte
// line m of each row), at byte g*8192 + dh*4096 + m*1024.  Inside block
// (g, dh, m), 16-byte position p holds the chunk (k-step j = 4m + (p >> 4),
// half hi = (p & 1) ^ (g & 1)) of row 8g + ((p >> 1) & 7), i.e. dims
// 16j + 8hi .. +8 of the dim half.  With this placement
//   * wave w copies rows 8w .. 8w+7, each copy instruction moving 8 whole
//     128-byte lines;
//   * the score operand of k-step j (lane: key l & 31, half l >> 5) sits at
//     a per-lane base + 256*j, conflict-free over every 16 lanes;
//   * the transposing PV reads sit at a per-lane base + 16384*pp + 512*mb,
//     conflict-free over every 16 lanes;
// so no LDS address arithmetic is left in the loop.
//
// The loop is software-pipelined with one barrier per tile: iteration i
// publishes the S partial of tile i, and after the barrier runs the PV
// product of tile i-1 and the score MFMAs of tile i+1 while tile i's softmax
// proceeds on the vector ALUs.  The S partials go through two exchange
// buffers used alternately (a buffer is rewritten only two barriers after
// it was read).  Tile i+3 is requested right after the barrier of iteration
// i, into the stage tile i-1 held, so two tiles are always in flight.  Q is
// loaded straight into registers, after the first metadata loads are issued
// so that its latency overlaps the metadata round trips.
//
// LDS: ring 4 x 32 KiB + exchange 2 x 16 KiB = 160 KiB; the prologue's slot
// list, per-tile key masks and page-table cache live in the exchange
// buffers until the loop starts.
// ---------------------------------------------------------------------------
template <int kHH, bool kDbg>
__global__ __launch_bounds__(256, 1) void attn_wide_kernel(AttnArgs a) {
    constexpr int kGroup = 4 / kHH;          // waves per head group (dim slices)
    constexpr int kDims = kHeadDim / kGroup;  // head dims per wave
    constexpr int kSteps = kDims / 16;        // score k-steps per tile
    constexpr int kMb = kDims / 32;           // PV dim blocks per wave
    constexpr int kHeads = 32 * kHH;          // heads per workgroup
    __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kStages][kTileKeys * 1024];
    __shared__ __attribute__((aligned(16))) float s_x[2][4 * 64 * 16];
    uint32_t* s_mask = (uint32_t*)&s_x[0][0];  // one 32-key mask per tile, prologue only
    int32_t* s_table = (int32_t*)&s_x[1][0];   // kTableCap entries, prologue only
    static_assert(kTableCap <= 4 * 64 * 16, "page-table cache fits buffer 1");

    fetch_args(a);
    Item it;
    const bool live = decode_item(a, it);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int hh = w / kGroup, dq = w % kGroup;

    // Round 1: the request bounds, the split's C4 indices and the guessed
    // request's extra page-table row, then Q (independent of all of them,
    // issued last so that waiting for the metadata does not wait for it).
    const RequestChunk rc = load_requests(a.m, 0, l);
    const int k0 = it.s * a.chunk;
    ExtPrefetch pf;
    prefetch_ext(a, it.t, k0, w, l, tid, pf);
    __builtin_amdgcn_sched_barrier(0);
    // Q^T as the B operand of the scores: lane holds head (l & 31) of the
    // wave's head group, dims kDims*dq + 16*j + 8*(l >> 5) .. +8 of k-step j.
    // Heads past H read head H-1; their results are never written.
    bf16x8 qf[kSteps];
    {
        const int my_head = it.hb * kHeads + hh * 32 + (l & 31);
        const uint16_t* qrow = a.q + (int64_t)it.t * a.q_s0 + (int64_t)min(my_head, a.H - 1) * a.q_s1 + dq * kDims + 8 * (l >> 5);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) qf[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * j));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!live) return;
    const RowKeys rk = row_keys_from(a.m, it.t, l, rc);
    const int n_here = __builtin_amdgcn_readfirstlane(max(0, min(rk.n_swa + rk.n_ext, k0 + a.chunk) - k0));
    const int n_tiles = (n_here + kTileKeys - 1) / kTileKeys;

    // Row addresses of the keys this wave copies: tile j, row 8w + e sits in
    // lane (8j + e) & 63 of ad[(8j + e) >> 6]; and, for the first three
    // tiles, the row lane l copies (8w + ((l >> 1) & 7)) in pro[j], so those
    // copies need no cross-lane step.  Unused keys read the zero row; window
    // keys are filled in once their page entries have arrived.
    const int dma_row = (l >> 1) & 7;
    uint64_t ad[kAdRegs], pro[3];
    {
        uint64_t addr[kLaneKeys];
        uint32_t valid;
        ext_addresses(a, rk, k0, n_here, w, l, tid, pf, s_table, addr, valid);
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) ad[u] = addr[u];
#pragma unroll
        for (int j = 0; j < 3; ++j) pro[j] = addr[kAdRegs + j];
        // Valid-key mask of every tile (byte w of word j: rows 8w .. 8w+7 of
        // tile j), published by the barrier before the first tile.
        uint8_t* s_mask8 = (uint8_t*)s_mask;
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) {
            const uint64_t b = __ballot((valid >> u) & 1u);
            if (l < 8) s_mask8[4 * (8 * u + l) + w] = (uint8_t)(b >> (8 * l));
        }
    }
    // Round 2 (window pages, scalar loads), issued after the last LDS access
    // above and waited for after the first copies below (nothing in between
    // touches LDS).
    __builtin_amdgcn_sched_barrier(0);
    SwaPages swp = issue_swa_pages(a, rk, k0, n_here);
    __builtin_amdgcn_sched_barrier(0);

    // Copy of one tile: lane p moves 16-byte chunks of row 8w + ((p >> 1) & 7),
    // at chunk 2*(p >> 4) + ((p & 1) ^ (w & 1)) of each 128-byte line, in four
    // parts of two lines each.  The row address comes from pro[] for the first
    // three tiles and from ad[] (one cross-lane permute) after them.
    const uint32_t dma_lane_off = 16u * (2u * (l >> 4) + ((l & 1) ^ (w & 1)));
    auto tile_row = [&](int tile) -> const uint8_t* {  // tile >= 3; past the split: zero rows
        const int u = min(tile >> 3, kMaxSplitKeys / 256 - 1);
        const uint64_t au = u == 0 ? ad[0] : (u == 1 ? ad[1] : (u == 2 ? ad[2] : ad[3]));
        const int src = 4 * (8 * (tile & 7) + dma_row);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)au);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(au >> 32));
        return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo) + dma_lane_off;
    };
    auto copy_part = [&](const uint8_t* row, int tile, auto part) {
        constexpr int kP = decltype(part)::value;
        const uint32_t dst = lds_addr(&s_tile[tile % kStages][0]) + w * 8192 + kP * 2048;
        dma16_off<256 * kP>(row, dst);
        dma16_off<256 * kP + 128>(row, dst + 1024);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    // Recording builds: lanes 0, 2, .., 14 (one per copied row, dma_row 0..7,
    // chunk offset 16*(w & 1)) record the row address of key 8*grp + dma_row
    // of the tile.
    auto dbg_row = [&](const uint8_t* row, int tile, int grp) {
        if constexpr (kDbg) {
            if ((l & 0x31) == 0)
                a.dbg_keys[dbg_unit(a, it) * a.chunk + kTileKeys * tile + 8 * grp + dma_row] =
                    (uint64_t)(uintptr_t)(row - dma_lane_off);
        }
    };
    auto fetch_tile = [&](int tile) {
        const uint8_t* row = tile < 3 ? (const uint8_t*)(uintptr_t)(tile == 0 ? pro[0] : (tile == 1 ? pro[1] : pro[2])) + dma_lane_off
                                      : tile_row(tile);
        dbg_row(row, tile, w);
        copy_part(row, tile, P0{});
        copy_part(row, tile, P1{});
        copy_part(row, tile, P2{});
        copy_part(row, tile, P3{});
    };

    // Per-lane LDS bases of the score operand and of the two transposing PV
    // reads (rows r0 = 16pp + 4hq + kq and r0 + 8); see the layout above.
    const int kk = l & 31, khi = l >> 5, kg = kk >> 3;
    const uint32_t s_base = kg * 8192 + dq * (16 * kDims) + 32 * (kk & 7) + 16 * (khi ^ (kg & 1));
    const int a4 = l & 3, kq = (l >> 2) & 3, half = (l >> 4) & 1, hq = l >> 5;
    const uint32_t t_base0 = dq * (16 * kDims) + 256 * half + 128 * hq + 32 * kq + 8 * a4;
    const uint32_t t_base1 = t_base0 + 8192 + 16 - 32 * (a4 >> 1);
    const uint32_t ring = lds_addr(&s_tile[0][0]);

    auto read_k = [&](int tile, bf16x8 (&av)[kSteps]) {
        const lds_void* base = (const lds_void*)(uintptr_t)(ring + (tile % kStages) * (kTileKeys * 1024) + s_base);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) av[j] = *(const __attribute__((address_space(3))) bf16x8*)((const __attribute__((address_space(3))) uint8_t*)base + 256 * j);
    };
    // K^T operand of PV: lane L takes dim 32*mb + (L & 31) of its dim slice
    // and keys G(pp, L >> 5) from two transposing reads (rows r0 and r0 + 8).
    auto read_kt = [&](int tile, bf16x8 (&kt)[2 * kMb]) {
        const uint32_t st = ring + (tile % kStages) * (kTileKeys * 1024);
        const __attribute__((address_space(3))) uint8_t* b0 = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + t_base0);
        const __attribute__((address_space(3))) uint8_t* b1 = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + t_base1);
#pragma unroll
        for (int mb = 0; mb < kMb; ++mb)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b0 + 16384 * pp + 512 * mb));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b1 + 16384 * pp + 512 * mb));
                kt[2 * mb + pp] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    };

    f32x16 oacc[kMb];
#pragma unroll
    for (int mb = 0; mb < kMb; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    // PV operands of the previous tile, consumed one iteration later (zero
    // before the first tile, so the first PV step adds nothing).
    bf16x8 kt[2 * kMb], pb[2];
#pragma unroll
    for (int j = 0; j < 2 * kMb; ++j) kt[j] = bf16x8{};
    pb[0] = bf16x8{};
    pb[1] = bf16x8{};

    // The tile copies below go out while Q (the last compiler-visible vector
    // loads) may still be in flight: every explicit vmcnt wait below counts
    // the copies issued after its target, and loads completing in order make
    // any earlier ones only strengthen it.
    // Tiles made of compressed entries only are requested right away.
    const int n_first = min(n_tiles, 3);
    const int n_early = min(n_first, max(0, rk.n_ext - k0) / kTileKeys);
    // Q has arrived by now (it was requested with the first metadata, a few
    // round trips ago).  Waiting for it here, before any tile copy (which the
    // compiler does not see), lets the compiler know it is in registers;
    // otherwise it would wait for it again before every score product of the
    // loop, and such a wait, counting the copies issued after Q as well,
    // would stall on the tiles still in flight.
    wait_vmcnt<0>();
    for (int j = 0; j < n_early; ++j) fetch_tile(j);
    __builtin_amdgcn_sched_barrier(0);
    wait_swa_pages(swp);
    __builtin_amdgcn_sched_barrier(0);
    // Window keys, now that their page entries have arrived.
    if (swp.any) {
        auto swa_addr = [&](int key, uint64_t cur) -> uint64_t {
            const int i = k0 + key;
            if (key >= n_here || i < rk.n_ext) return cur;
            const int x = rk.swa_lo + (i - rk.n_ext);
            const int pk = (x >> 8) - swp.pg_lo;
            const int32_t e = pk == 0 ? swp.e[0] : (pk == 1 ? swp.e[1] : (pk == 2 ? swp.e[2] : (pk == 3 ? swp.e[3] : swp.e[4])));
            return (uint64_t)(uintptr_t)(a.swa_pool + ((int64_t)e * kPage + (x & (kPage - 1))) * a.swa_row_bytes);
        };
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) {
            const int idx = 64 * u + l;
            ad[u] = swa_addr(kTileKeys * (idx >> 3) + 8 * w + (idx & 7), ad[u]);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) pro[j] = swa_addr(kTileKeys * j + 8 * w + dma_row, pro[j]);
    }
    for (int j = n_early; j < n_first; ++j) fetch_tile(j);
    __syncthreads();  // tile masks published
    const uint32_t tile_mask = s_mask[l & 31];  // lane j: valid keys of tile j
    if constexpr (kDbg) {
        if (w == 0 && l < n_tiles) a.dbg_masks[dbg_unit(a, it) * 32 + l] = tile_mask;
    }
    f32x16 sacc = f32x16{};
    if (n_tiles > 0) {
        if (n_tiles > 2) wait_vmcnt<16>();
        else if (n_tiles > 1) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        __syncthreads();  // tile 0 is in LDS for every wave; the prologue scratch is dead
        bf16x8 av[kSteps];
        read_k(0, av);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], qf[j], sacc, 0, 0, 0);
    }

    const float sl2 = a.scale_log2;
    const int key_shift = 4 * khi;  // register r of a score tile: key 8*(r >> 2) + 4*(l >> 5) + (r & 3)
    // One iteration; kFetch: tile i+3 exists and is requested, its copy split
    // into four parts spread over the iteration (a burst of copies would hold
    // the wave at the memory queue), from a row address computed one
    // iteration ahead.
    const uint8_t* next_row = tile_row(3);
    auto iteration = [&](int i, auto fetch_tag) {
        constexpr bool kFetch = decltype(fetch_tag)::value;
        // This wave's rows of tile i+1 (tile i+2 may still be in flight).
        if (kFetch || i + 2 < n_tiles) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        float* xb = &s_x[i & 1][0];
        {
            f32x4* mine = (f32x4*)xb + w * 256 + l;
#pragma unroll
            for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
        }
        __syncthreads();  // S partials of tile i published; tile i+1 landed; tile i-1's stage is free
        const uint8_t* row = next_row;
        if constexpr (kFetch) next_row = tile_row(i + 4);

        // The other S partials of the head group for tile i (the waves that
        // hold the other dim slices: dq ^ 1, and for four slices dq ^ 2 and
        // dq ^ 3) and the score operand of tile i+1 (when tile i is the last,
        // that stage holds stale rows whose scores are discarded).
        f32x4 part[kGroup - 1][4];
#pragma unroll
        for (int v = 1; v < kGroup; ++v) {
            const f32x4* op = (const f32x4*)xb + (hh * kGroup + (dq ^ v)) * 256 + l;
#pragma unroll
            for (int q = 0; q < 4; ++q) part[v - 1][q] = op[64 * q];
        }
        bf16x8 av[kSteps];
        read_k(i + 1, av);
        if constexpr (kFetch) {
            dbg_row(row, i + 3, w);
            copy_part(row, i + 3, P0{});
        }

        // PV of tile i-1 (operands from the previous iteration), interleaved
        // with the first half of tile i's softmax.  Register r of a score tile
        // holds head (l & 31), key 8*(r >> 2) + 4*(l >> 5) + (r & 3); lanes l and
        // l ^ 32 hold the two halves of a head's keys.  The scores of the head
        // group are the sum of its dim slices' partials, added pairwise
        // ((slices 0+1) + (slices 2+3)) so that every wave of the group gets
        // the same value (each addition is commutative).
#pragma unroll
        for (int mb = 0; mb < kMb; ++mb)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[2 * mb + pp], pb[pp], oacc[mb], 0, 0, 0);
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float own = sacc[r] + part[0][r >> 2][r & 3];
            if constexpr (kGroup == 2) {
                sv[r] = own;
            } else {
                sv[r] = own + (part[1][r >> 2][r & 3] + part[2][r >> 2][r & 3]);
            }
        }
        {
            const uint32_t tm = (uint32_t)__builtin_amdgcn_readlane((int)tile_mask, i);
            if (tm != 0xFFFFFFFFu) {  // a tile with unused keys (uniform)
                const uint32_t mine = tm >> key_shift;
#pragma unroll
                for (int r = 0; r < 16; ++r) sv[r] = ((mine >> (8 * (r >> 2) + (r & 3))) & 1u) ? sv[r] : -INFINITY;
            }
        }
        float smax = sv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) smax = fmaxf(smax, sv[r]);
        const float tmax = smax * sl2;  // scale > 0: the maximum commutes with it
#pragma unroll
        for (int j = 0; j < 2 * kMb; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);  // then VALU / transcendental
        }
        if constexpr (kFetch) copy_part(row, i + 3, P1{});

        // The running reference m_run (scaled units) moves only when a score
        // exceeds it by more than 2^8 (probabilities stay <= 256), so the
        // accumulators are rescaled on few tiles (after the PV product above,
        // which used the old reference); l_run is this lane's share of the
        // denominator, the two shares are added in write_result.
        if (__any(tmax > m_run + kRescaleLog2)) {
            const float hmax = fmaxf(tmax, __shfl_xor(tmax, 32));  // the head's tile maximum
            const bool grow = hmax > m_run + kRescaleLog2;
            const float m_target = grow ? hmax : m_run;
            const float alpha = fast_exp2(m_run - m_target);  // 0 while nothing was accumulated
            if (__any(grow && m_run != -INFINITY)) scale_accumulators(oacc, alpha);
            l_run *= alpha;
            m_run = m_target;
        }
        // The PV operand of tile i (its stage is read for the last time).
        read_kt(i, kt);
        if constexpr (kFetch) {
            copy_part(row, i + 3, P2{});
            copy_part(row, i + 3, P3{});
        }

        // Second half of the softmax (base 2, raw scores; the scale is applied
        // in the exponent), interleaved with the score MFMAs of tile i+1.
        f32x16 snext = f32x16{};
#pragma unroll
        for (int j = 0; j < kSteps; ++j) snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], qf[j], snext, 0, 0, 0);
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(fmaf(sv[r], sl2, neg_m));
            psum += pr;
            pb[r >> 3][r & 7] = (__bf16)pr;
        }
        l_run += psum;
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // then VALU / transcendental
        }
        sacc = snext;
    };
    int i = 0;
    for (; i + 3 < n_tiles; ++i) iteration(i, std::true_type{});
    for (; i < n_tiles; ++i) iteration(i, std::false_type{});
    // PV of the last tile.
#pragma unroll
    for (int mb = 0; mb < kMb; ++mb)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
            oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[2 * mb + pp], pb[pp], oacc[mb], 0, 0, 0);
    write_result<kHH>(a, it, hh, dq, l, oacc, m_run, l_run, &s_tile[0][0], &s_tile[1][0]);
}

// ---------------------------------------------------------------------------
// bf16 KV, one workgroup per (query row, block of 32 heads, key split), with
// the four waves in two roles.  Waves 0 and 1 (score waves) compute the
// scores of every head of the block over dim half d = w and the softmax;
// waves 2 and 3 (PV waves) accumulate O for every head of the block over dim
// half d = w - 2.  Each key operand is therefore read from LDS by one wave
// per dim half only (the score operand by a score wave, the transposing
// PV operand by a PV wave), half of what a split by heads reads.  Key rows
// stream from HBM into a 4-stage LDS ring with direct global->LDS copies:
// the first three tiles by all four waves (8 rows each), the later ones by
// the PV waves alone (16 rows each: their own and the score wave's of the
// same parity), so that the score waves never wait at the memory queue
// inside the loop (measured slightly faster than each wave copying its own
// rows).
//
// Tile layout in LDS (32 KiB per stage): as for the score and transposing
// reads of the dim-half kernels -- rows 8g .. 8g+7 form group g; the 512
// bytes of dim half d of those rows form four 1 KiB blocks m (128-byte line
// m of each row) at byte g*8192 + d*4096 + m*1024; inside a block, 16-byte
// position p holds the chunk (k-step 4m + (p >> 4), half (p & 1) ^ (g & 1))
// of row 8g + ((p >> 1) & 7).
//
// Pipeline, one barrier per tile.  Iteration i:
//   score waves publish their score partial of tile i (all 32 heads, their
//   dim half), and P and the rescale factors of tile i-1; after the barrier
//   each reads both partials of its 16 heads (the block's heads are split
//   between the two score waves for the softmax), runs tile i's softmax on
//   their sum, interleaved with the score products of tile i+1;
//   PV waves, after the barrier, request tile i+3, read P of tile i-1,
//   rescale their accumulators if the reference moved, run the PV product of
//   tile i-1 and read the PV operand of tile i (held in registers until the
//   next iteration, so tile i's stage is free at barrier i+1).
//
// LDS: ring 4 x 32 KiB + 2 exchange buffers (two 4.5 KiB partials, 2 KiB of
// P, the factors); the prologue's page-table cache, tile masks and the score
// waves' row addresses live in the exchange buffers until the loop starts.
// ---------------------------------------------------------------------------
template <int kHH, bool kDbg>
__global__ __launch_bounds__(256, 1) void attn_ws_kernel(AttnArgs a) {
    constexpr int kDims = kHeadDim / 2;  // head dims per wave (a dim half)
    constexpr int kSteps = kDims / 16;   // score k-steps per tile
    constexpr int kMb = kDims / 32;      // PV dim blocks per wave
    constexpr int kHeads = 32 * kHH;     // heads per workgroup
    static_assert(kHH == 1, "the score waves' softmax layout covers one 32-head block");
    // Exchange buffer: the two score partials (partial d: fp32 [32 heads][32
    // keys], rows padded to 144 bytes so that 16 consecutive rows start in
    // distinct banks), then P in the PV operand layout (64 lanes x 32 bytes),
    // the rescale factor of each head, and at the end the output scales.
    constexpr int kRowBytes = 144;
    constexpr int kPartBytes = 32 * kRowBytes;
    constexpr int kXP = 2 * kPartBytes;                   // P
    constexpr int kXF = kXP + 2048;                       // factor of head j at kXF + 4j
    constexpr int kXBytes = kXF + 128 + 128;              // + the output scales at the end
    __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kStages][kTileKeys * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kXBytes];
    uint32_t* s_mask = (uint32_t*)&s_x[0][0];  // one 32-key mask per tile, prologue only
    int32_t* s_table = (int32_t*)&s_x[1][0];   // kTableCap entries, prologue only
    static_assert(kTableCap * 4 <= kXBytes, "page-table cache fits buffer 1");
    constexpr int kAdOffset = kTableCap * 4;  // score waves' row addresses in buffer 1, prologue only
    static_assert(kAdOffset + 2 * kAdRegs * 64 * 8 <= kXBytes, "row addresses fit buffer 1");

    fetch_args(a);
    Item it;
    const bool live = decode_item(a, it);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int d = w & 1;          // dim half of the wave's products
    const bool score = w < 2;     // score wave (else PV wave), wave-uniform

    // Round 1: the request bounds, the split's C4 indices and the guessed
    // request's extra page-table row, then Q (independent of all of them,
    // issued last so that waiting for the metadata does not wait for it).
    const RequestChunk rc = load_requests(a.m, 0, l);
    const int k0 = it.s * a.chunk;
    ExtPrefetch pf;
    prefetch_ext(a, it.t, k0, w, l, tid, pf);
    __builtin_amdgcn_sched_barrier(0);
    // Score waves: Q^T as the B operand of the scores (lane: head l & 31,
    // dims 256*d + 16*j + 8*(l >> 5) .. +8 of k-step j).  Heads past H read
    // head H-1; their results are never written.  PV waves load no Q.
    bf16x8 qf[kSteps];
    float sink_raw = 0.f;  // the sink logit of the head of this lane's softmax (read early: it ends the chain)
    if (score) {
        const int sink_head = min(it.hb * kHeads + 16 * d + (l & 15), a.H - 1);
        sink_raw = *(a.sink != nullptr ? a.sink + sink_head : (const float*)a.zero_row);
        const int my_head = it.hb * kHeads + (l & 31);
        const uint16_t* qrow = a.q + (int64_t)it.t * a.q_s0 + (int64_t)min(my_head, a.H - 1) * a.q_s1 + d * kDims + 8 * (l >> 5);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) qf[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * j));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!live) return;
    const RowKeys rk = row_keys_from(a.m, it.t, l, rc);
    const int n_here = __builtin_amdgcn_readfirstlane(max(0, min(rk.n_swa + rk.n_ext, k0 + a.chunk) - k0));
    const int n_tiles = (n_here + kTileKeys - 1) / kTileKeys;

    // Row addresses of the keys this wave copies: tile j, row 8w + e sits in
    // lane (8j + e) & 63 of ad[(8j + e) >> 6]; and, for the first three
    // tiles, the row lane l copies (8w + ((l >> 1) & 7)) in pro[j], so those
    // copies need no cross-lane step.  Unused keys read the zero row; window
    // keys are filled in once their page entries have arrived.
    const int dma_row = (l >> 1) & 7;
    uint64_t ad[kAdRegs], pro[3];
    {
        uint64_t addr[kLaneKeys];
        uint32_t valid;
        ext_addresses(a, rk, k0, n_here, w, l, tid, pf, s_table, addr, valid);
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) ad[u] = addr[u];
#pragma unroll
        for (int j = 0; j < 3; ++j) pro[j] = addr[kAdRegs + j];
        // Valid-key mask of every tile (byte w of word j: rows 8w .. 8w+7 of
        // tile j), published by the barrier before the first tile.
        uint8_t* s_mask8 = (uint8_t*)s_mask;
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) {
            const uint64_t b = __ballot((valid >> u) & 1u);
            if (l < 8) s_mask8[4 * (8 * u + l) + w] = (uint8_t)(b >> (8 * l));
        }
    }
    // Round 2 (window pages, scalar loads), issued after the last LDS access
    // above and waited for after the first copies below (nothing in between
    // touches LDS).
    __builtin_amdgcn_sched_barrier(0);
    SwaPages swp = issue_swa_pages(a, rk, k0, n_here);
    __builtin_amdgcn_sched_barrier(0);

    // Copy of one tile: lane p moves 16-byte chunks of row 8w + ((p >> 1) & 7),
    // at chunk 2*(p >> 4) + ((p & 1) ^ (w & 1)) of each 128-byte line, in four
    // parts of two lines each.  The row address comes from pro[] for the first
    // three tiles and from ad[] (one cross-lane permute) after them.
    const uint32_t dma_lane_off = 16u * (2u * (l >> 4) + ((l & 1) ^ (w & 1)));
    auto tile_row = [&](int tile) -> const uint8_t* {  // tile >= 3; past the split: zero rows
        const int u = min(tile >> 3, kMaxSplitKeys / 256 - 1);
        const uint64_t au = u == 0 ? ad[0] : (u == 1 ? ad[1] : (u == 2 ? ad[2] : ad[3]));
        const int src = 4 * (8 * (tile & 7) + dma_row);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)au);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(au >> 32));
        return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo) + dma_lane_off;
    };
    auto copy_part = [&](const uint8_t* row, int tile, auto part) {
        constexpr int kP = decltype(part)::value;
        const uint32_t dst = lds_addr(&s_tile[tile % kStages][0]) + w * 8192 + kP * 2048;
        dma16_off<256 * kP>(row, dst);
        dma16_off<256 * kP + 128>(row, dst + 1024);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    // Recording builds: lanes 0, 2, .., 14 (one per copied row, dma_row 0..7,
    // chunk offset 16*(w & 1)) record the row address of key 8*grp + dma_row
    // of the tile.
    auto dbg_row = [&](const uint8_t* row, int tile, int grp) {
        if constexpr (kDbg) {
            if ((l & 0x31) == 0)
                a.dbg_keys[dbg_unit(a, it) * a.chunk + kTileKeys * tile + 8 * grp + dma_row] =
                    (uint64_t)(uintptr_t)(row - dma_lane_off);
        }
    };
    auto fetch_tile = [&](int tile) {
        const uint8_t* row = tile < 3 ? (const uint8_t*)(uintptr_t)(tile == 0 ? pro[0] : (tile == 1 ? pro[1] : pro[2])) + dma_lane_off
                                      : tile_row(tile);
        dbg_row(row, tile, w);
        copy_part(row, tile, P0{});
        copy_part(row, tile, P1{});
        copy_part(row, tile, P2{});
        copy_part(row, tile, P3{});
    };

    // Per-lane LDS bases of the score operand and of the two transposing PV
    // reads (rows r0 = 16pp + 4hq + kq and r0 + 8); see the layout above.
    const int kk = l & 31, khi = l >> 5, kg = kk >> 3;
    const uint32_t s_base = kg * 8192 + d * (16 * kDims) + 32 * (kk & 7) + 16 * (khi ^ (kg & 1));
    const int a4 = l & 3, kq = (l >> 2) & 3, half = (l >> 4) & 1, hq = l >> 5;
    const uint32_t t_base0 = d * (16 * kDims) + 256 * half + 128 * hq + 32 * kq + 8 * a4;
    const uint32_t t_base1 = t_base0 + 8192 + 16 - 32 * (a4 >> 1);
    const uint32_t ring = lds_addr(&s_tile[0][0]);

    auto read_k = [&](int tile, bf16x8 (&av)[kSteps]) {
        const lds_void* base = (const lds_void*)(uintptr_t)(ring + (tile % kStages) * (kTileKeys * 1024) + s_base);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) av[j] = *(const __attribute__((address_space(3))) bf16x8*)((const __attribute__((address_space(3))) uint8_t*)base + 256 * j);
    };
    // Half of the score operand (k-steps 8h .. 8h+7), for the two-block
    // score waves, which cannot hold all sixteen k-steps besides Q.
    auto read_k_half = [&](int tile, int h, bf16x8 (&av)[kSteps / 2]) {
        const lds_void* base = (const lds_void*)(uintptr_t)(ring + (tile % kStages) * (kTileKeys * 1024) + s_base + 2048 * h);
#pragma unroll
        for (int j = 0; j < kSteps / 2; ++j) av[j] = *(const __attribute__((address_space(3))) bf16x8*)((const __attribute__((address_space(3))) uint8_t*)base + 256 * j);
    };
    // K^T operand of PV: lane L takes dim 32*mb + (L & 31) of its dim slice
    // and keys G(pp, L >> 5) from two transposing reads (rows r0 and r0 + 8).
    auto read_kt = [&](int tile, bf16x8 (&kt)[2 * kMb]) {
        const uint32_t st = ring + (tile % kStages) * (kTileKeys * 1024);
        const __attribute__((address_space(3))) uint8_t* b0 = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + t_base0);
        const __attribute__((address_space(3))) uint8_t* b1 = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + t_base1);
#pragma unroll
        for (int mb = 0; mb < kMb; ++mb)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b0 + 16384 * pp + 512 * mb));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b1 + 16384 * pp + 512 * mb));
                kt[2 * mb + pp] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    };


    auto xbuf = [&](int i) -> uint8_t* { return &s_x[i & 1][0]; };

    // The tile copies below go out while Q (the last compiler-visible vector
    // loads) may still be in flight: every explicit vmcnt wait below counts
    // the copies issued after its target, and loads completing in order make
    // any earlier ones only strengthen it.
    // Tiles made of compressed entries only are requested right away.
    const int n_first = min(n_tiles, 3);
    const int n_early = min(n_first, max(0, rk.n_ext - k0) / kTileKeys);
    // Q has arrived by now (it was requested with the first metadata, a few
    // round trips ago).  Waiting for it here, before any tile copy (which the
    // compiler does not see), lets the compiler know it is in registers;
    // otherwise it would wait for it again before every score product of the
    // loop, and such a wait, counting the copies issued after Q as well,
    // would stall on the tiles still in flight.
    wait_vmcnt<0>();
    for (int j = 0; j < n_early; ++j) fetch_tile(j);
    __builtin_amdgcn_sched_barrier(0);
    wait_swa_pages(swp);
    __builtin_amdgcn_sched_barrier(0);
    // Window keys, now that their page entries have arrived.
    if (swp.any) {
        auto swa_addr = [&](int key, uint64_t cur) -> uint64_t {
            const int i = k0 + key;
            if (key >= n_here || i < rk.n_ext) return cur;
            const int x = rk.swa_lo + (i - rk.n_ext);
            const int pk = (x >> 8) - swp.pg_lo;
            const int32_t e = pk == 0 ? swp.e[0] : (pk == 1 ? swp.e[1] : (pk == 2 ? swp.e[2] : (pk == 3 ? swp.e[3] : swp.e[4])));
            return (uint64_t)(uintptr_t)(a.swa_pool + ((int64_t)e * kPage + (x & (kPage - 1))) * a.swa_row_bytes);
        };
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) {
            const int idx = 64 * u + l;
            ad[u] = swa_addr(kTileKeys * (idx >> 3) + 8 * w + (idx & 7), ad[u]);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) pro[j] = swa_addr(kTileKeys * j + 8 * w + dma_row, pro[j]);
    }
    for (int j = n_early; j < n_first; ++j) fetch_tile(j);
    // The score waves' row addresses of tiles 3 and later, for the PV wave
    // that copies those rows in the loop (in buffer 1, past the page-table
    // cache; the buffer's first use in the loop follows the barrier of
    // iteration 0, by which the PV waves have read them).
    uint64_t* const s_ad = (uint64_t*)(&s_x[1][0] + kAdOffset);
    if (score) {
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) s_ad[(d * kAdRegs + u) * 64 + l] = ad[u];
    }
    __syncthreads();  // tile masks and the score waves' row addresses published
    const uint32_t tile_mask = s_mask[l & 31];  // lane j: valid keys of tile j
    if constexpr (kDbg) {
        if (w == 0 && l < n_tiles) a.dbg_masks[dbg_unit(a, it) * 32 + l] = tile_mask;
    }
    if (n_tiles > 0) {
        if (n_tiles > 2) wait_vmcnt<16>();
        else if (n_tiles > 1) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        __syncthreads();  // tile 0 is in LDS for every wave; the prologue scratch is dead
    }
    const uint8_t* next_row = tile_row(3);
    uint8_t* const xb_end = xbuf(n_tiles);
    float* const s_f = (float*)(xb_end + kXF + 128);  // output scale of head j of the block, at the end

    // The two roles run separate loops (so that the compiler allocates each
    // role's registers on its own); each loop has exactly one barrier per
    // tile.  Only the PV waves copy tiles in the loop.
    if (score) {
        // Scores: wave d computes the partial over dim half d for all 32
        // heads (MFMA layout: register r of lane l holds head l & 31, key
        // 8*(r >> 2) + 4*(l >> 5) + (r & 3)), and publishes it.  The softmax
        // then runs on the sum of both partials in another layout, which
        // splits the block's heads between the two waves: lane l of wave d
        // holds head hs = 16d + (l & 15) and keys 8g .. 8g+7, g = l >> 4, so
        // each wave exponentiates half of the tile.
        const float sl2 = a.scale_log2;
        const int hs = 16 * d + (l & 15), g = l >> 4;
        float m_run = -INFINITY, l_run = 0.f;  // per head (the same in its four lanes); l_run: this lane's keys
        f32x16 sacc = f32x16{};
        if (n_tiles > 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 av[kSteps / 2];
                read_k_half(0, h, av);
#pragma unroll
                for (int j = 0; j < kSteps / 2; ++j)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], qf[8 * h + j], sacc, 0, 0, 0);
            }
        }
        // P of a tile for the PV waves: keys 8g .. 8g+3 of head hs go to PV
        // lane hs, keys 8g+4 .. 8g+7 to PV lane hs + 32, both at k-step g >> 1,
        // elements 4*(g & 1) .. +3 (see pv_step).
        u32x2 p_lo = u32x2{0u, 0u}, p_hi = u32x2{0u, 0u};
        float alpha_out = 1.f;
        // Publish this wave's partial of tile i and its heads' P and rescale
        // factors of tile i-1.
        auto publish = [&](uint8_t* xb, bool with_partial, bool with_p) __attribute__((always_inline)) {
            if (with_partial) {
                // Row: head l & 31; keys 4c .. 4c+3 (c = 2q + (l >> 5)) at byte 16c.
                uint8_t* row = xb + d * kPartBytes + (l & 31) * kRowBytes + 16 * (l >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(f32x4*)(row + 32 * q) = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
            }
            if (with_p) {
                uint8_t* pb = xb + kXP + 16 * (g >> 1) + 8 * (g & 1);
                *(u32x2*)(pb + 32 * hs) = p_lo;
                *(u32x2*)(pb + 32 * (hs + 32)) = p_hi;
                if (l < 16) ((float*)(xb + kXF))[hs] = alpha_out;
            }
        };
        auto iteration = [&](int i) __attribute__((always_inline)) {
            // This wave's rows of tile i+1 if it copied them (tiles 1 and 2;
            // tile 2 may still be in flight at tile 0).
            if (i == 0 && n_tiles > 2) wait_vmcnt<8>();
            else wait_vmcnt<0>();
            uint8_t* xb = xbuf(i);
            publish(xb, true, i > 0);
            __syncthreads();  // partials of tile i, P of tile i-1 published; tile i+1 landed; tile i-1's stage is free
            // Both partials of this lane's keys of tile i, and the score
            // operand of tile i+1 (when tile i is the last, that stage holds
            // stale rows whose scores are discarded).
            f32x4 pa[2], pb2[2];
            {
                const uint8_t* r0 = xb + hs * kRowBytes + 32 * g;
                pa[0] = *(const f32x4*)(r0);
                pa[1] = *(const f32x4*)(r0 + 16);
                pb2[0] = *(const f32x4*)(r0 + kPartBytes);
                pb2[1] = *(const f32x4*)(r0 + kPartBytes + 16);
            }
            bf16x8 av[kSteps];
            read_k(i + 1, av);
            // Score products of tile i+1 in two halves: the first interleaved
            // with tile i's sums, mask and maximum, the second (after the
            // rescale decision) with its exponentials.
            f32x16 snext = f32x16{};
            constexpr int kHalf = kSteps / 2;
#pragma unroll
            for (int j = 0; j < kHalf; ++j) snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], qf[j], snext, 0, 0, 0);
            float sv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) sv[k] = pa[k >> 2][k & 3] + pb2[k >> 2][k & 3];
            {
                const uint32_t tm = (uint32_t)__builtin_amdgcn_readlane((int)tile_mask, i);
                if (tm != 0xFFFFFFFFu) {  // a tile with unused keys (uniform)
                    const uint32_t mine = tm >> (8 * g);
#pragma unroll
                    for (int k = 0; k < 8; ++k) sv[k] = ((mine >> k) & 1u) ? sv[k] : -INFINITY;
                }
            }
            float smax = sv[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) smax = fmaxf(smax, sv[k]);
            const float tmax = smax * sl2;  // scale > 0: the maximum commutes with it
#pragma unroll
            for (int j = 0; j < kHalf; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);  // then VALU
            }
            // The running reference m_run (scaled units) moves only when a
            // score exceeds it by more than 2^8 (probabilities stay <= 256);
            // the PV waves rescale their accumulators by the factor published
            // with this tile's P.
            alpha_out = 1.f;
            if (__any(tmax > m_run + kRescaleLog2)) {
                float hmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                hmax = fmaxf(hmax, __shfl_xor(hmax, 32));  // the head's tile maximum (its four lanes)
                const bool grow = hmax > m_run + kRescaleLog2;
                const float m_target = grow ? hmax : m_run;
                const float alpha = fast_exp2(m_run - m_target);  // 0 while nothing was accumulated
                l_run *= alpha;
                alpha_out = m_run == -INFINITY ? 1.f : alpha;  // nothing accumulated yet: nothing to rescale
                m_run = m_target;
            }
#pragma unroll
            for (int j = 0; j < kHalf; ++j)
                snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kHalf + j], qf[kHalf + j], snext, 0, 0, 0);
            const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
            float pr[8];
            float psum = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = fast_exp2(fmaf(sv[k], sl2, neg_m));
                psum += pr[k];
            }
            l_run += psum;
            p_lo = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
            p_hi = u32x2{pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
#pragma unroll
            for (int j = 0; j < kHalf; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);  // then VALU / transcendental
            }
            sacc = snext;
        };
        for (int i = 0; i < n_tiles; ++i) iteration(i);

        // The last tile's P, the output scale of every head and lse.
        if (n_tiles > 0) publish(xb_end, false, true);
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);  // all 32 keys of the head
        const int my_head = it.hb * kHeads + hs;
        const bool head_ok = my_head < a.H;
        float f = 0.f, lse2 = -INFINITY;
        if (a.splits == 1) {
            const float sig = a.sink != nullptr && head_ok ? sink_raw * kLog2e : -INFINITY;
            const float M = fmaxf(m_run, sig);
            if (M != -INFINITY) {
                const float em = fast_exp2(m_run - M);
                const float den = l_tot * em + fast_exp2(sig - M);
                f = em / den;
                lse2 = M + fast_log2(den);
            }
        } else if (l_tot > 0.f) {
            f = 1.f / l_tot;
            lse2 = m_run + fast_log2(l_tot);
        }
        if (l < 16) {
            s_f[hs] = f;
            if (head_ok) {
                if (a.splits == 1) {
                    if (a.lse != nullptr) a.lse[(int64_t)it.t * a.lse_s0 + my_head] = lse2 * kLn2;
                } else {
                    a.ws_lse[((int64_t)it.t * a.splits + it.s) * a.H + my_head] = lse2;
                }
            }
        }
        __syncthreads();  // last P and the output scales published; every wave is done with the ring
    } else {
        // Accumulators of every head block over dim half d, and the PV
        // operand of the previous tile.
        f32x16 oacc[kHH][kMb];
#pragma unroll
        for (int hb = 0; hb < kHH; ++hb)
#pragma unroll
            for (int mb = 0; mb < kMb; ++mb) oacc[hb][mb] = f32x16{};
        bf16x8 kt[2 * kMb];
        // P of a tile (published in xb) times its operand, after the rescale
        // the softmax asked for.
        auto pv_step = [&](const uint8_t* xb) __attribute__((always_inline)) {
#pragma unroll
            for (int hb = 0; hb < kHH; ++hb) {
                const bf16x8* pp = (const bf16x8*)(xb + kXP) + 2 * l;
                const bf16x8 p0 = pp[0], p1 = pp[1];
                const float alpha = ((const float*)(xb + kXF))[l & 31];
                if (__any(alpha != 1.f)) scale_accumulators(oacc[hb], alpha);
#pragma unroll
                for (int mb = 0; mb < kMb; ++mb) {
                    oacc[hb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[2 * mb], p0, oacc[hb][mb], 0, 0, 0);
                    oacc[hb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[2 * mb + 1], p1, oacc[hb][mb], 0, 0, 0);
                }
            }
        };
        // The score wave of the same parity (whose rows this wave copies from
        // tile 3 on, with the same lane offsets): its row addresses, and its
        // copy of one tile part, into its rows' place in the stage.
        uint64_t ad_s[kAdRegs];
#pragma unroll
        for (int u = 0; u < kAdRegs; ++u) ad_s[u] = s_ad[(d * kAdRegs + u) * 64 + l];
        auto tile_row_s = [&](int tile) -> const uint8_t* {
            const int u = min(tile >> 3, kMaxSplitKeys / 256 - 1);
            const uint64_t au = u == 0 ? ad_s[0] : (u == 1 ? ad_s[1] : (u == 2 ? ad_s[2] : ad_s[3]));
            const int src = 4 * (8 * (tile & 7) + dma_row);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)au);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(au >> 32));
            return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo) + dma_lane_off;
        };
        auto copy_part_s = [&](const uint8_t* row, int tile, auto part) {
            constexpr int kP = decltype(part)::value;
            const uint32_t dst = lds_addr(&s_tile[tile % kStages][0]) + d * 8192 + kP * 2048;
            dma16_off<256 * kP>(row, dst);
            dma16_off<256 * kP + 128>(row, dst + 1024);
        };
        const uint8_t* next_row_s = tile_row_s(3);
        auto iteration = [&](int i, auto fetch_tag, auto first_tag) __attribute__((always_inline)) {
            constexpr bool kFetch = decltype(fetch_tag)::value;
            constexpr bool kFirst = decltype(first_tag)::value;  // i == 0: no earlier tile to multiply
            // Tile i+1 (copies of tile i+2 may still be in flight: 8 for tile
            // 2, from the prologue; 16 for a later one).
            if (i + 2 < n_tiles) {
                if (i == 0) wait_vmcnt<8>();
                else wait_vmcnt<16>();
            } else {
                wait_vmcnt<0>();
            }
            const uint8_t* xb = xbuf(i);
            __syncthreads();  // see the score waves' loop
            const uint8_t* row = next_row;
            const uint8_t* row_s = next_row_s;
            if constexpr (kFetch) {
                next_row = tile_row(i + 4);
                next_row_s = tile_row_s(i + 4);
                dbg_row(row, i + 3, w);
                dbg_row(row_s, i + 3, d);
                copy_part(row, i + 3, P0{});
                copy_part_s(row_s, i + 3, P0{});
                copy_part(row, i + 3, P1{});
                copy_part_s(row_s, i + 3, P1{});
            }
            if constexpr (!kFirst) pv_step(xb);  // tile i-1, with its operand read last iteration
            if constexpr (kFetch) {
                copy_part(row, i + 3, P2{});
                copy_part_s(row_s, i + 3, P2{});
                copy_part(row, i + 3, P3{});
                copy_part_s(row_s, i + 3, P3{});
            }
            read_kt(i, kt);  // tile i (landed at barrier i-1): its stage is read for the last time
        };
        // Iteration 0 is peeled (no PV product yet), so that every loop
        // iteration runs the product unconditionally: a path around it would
        // make the compiler copy all accumulators out of the AGPRs on every
        // iteration, for the loop's exit.
        int i = 0;
        if (n_tiles > 3) iteration(0, std::true_type{}, std::true_type{});
        else if (n_tiles > 0) iteration(0, std::false_type{}, std::true_type{});
        for (i = 1; i + 3 < n_tiles; ++i) iteration(i, std::true_type{}, std::false_type{});
        for (; i < n_tiles; ++i) iteration(i, std::false_type{}, std::false_type{});

        __syncthreads();  // see the score waves
        if (n_tiles > 0) pv_step(xb_end);
        // The unscaled fp32 rows, straight from the accumulators, into the
        // ring (free now): O^T register r of dim block mb holds dim 256*d +
        // 32*mb + 8*(r >> 2) + 4*(l >> 5) + (r & 3) of head l & 31, i.e. 16-byte
        // chunk c = 64d + 8mb + 2(r >> 2) + (l >> 5) of the head's 2 KiB row,
        // stored at chunk c ^ (head & 15) (conflict-free over 16 heads).  The
        // scaling and the conversion are left to all four waves below.
        const int r = l & 31;
        uint8_t* base = &s_tile[0][0] + r * 2048;
#pragma unroll
        for (int mb = 0; mb < kMb; ++mb) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int c = 64 * d + 8 * mb + 2 * qd + (l >> 5);
                const f32x16& o = oacc[0][mb];
                *(f32x4*)(base + 16 * (c ^ (r & 15))) = f32x4{o[4 * qd], o[4 * qd + 1], o[4 * qd + 2], o[4 * qd + 3]};
            }
        }
    }
    __syncthreads();  // rows staged
    // Wave w scales, converts and stores rows w*kRows .. +kRows (heads past H
    // skipped); lane l takes dims 8l .. 8l+7 (chunks 2l, 2l+1) of a row.  All
    // LDS reads go out first.
    constexpr int kRows = kHeads / 4;
    u32x4 v[kRows];
    {
        f32x4 x[kRows][2];
        float f[kRows];
#pragma unroll
        for (int e = 0; e < kRows; ++e) {
            const int r = kRows * w + e;
            const uint8_t* row = &s_tile[0][0] + r * 2048;
            x[e][0] = *(const f32x4*)(row + 16 * ((2 * l) ^ (r & 15)));
            x[e][1] = *(const f32x4*)(row + 16 * ((2 * l + 1) ^ (r & 15)));
            f[e] = s_f[r];
        }
#pragma unroll
        for (int e = 0; e < kRows; ++e)
            v[e] = u32x4{pack_bf16x2(x[e][0][0] * f[e], x[e][0][1] * f[e]), pack_bf16x2(x[e][0][2] * f[e], x[e][0][3] * f[e]),
                         pack_bf16x2(x[e][1][0] * f[e], x[e][1][1] * f[e]), pack_bf16x2(x[e][1][2] * f[e], x[e][1][3] * f[e])};
    }
    const int head0 = it.hb * kHeads + kRows * w;
    const int n_rows = min(kRows, a.H - head0);  // uniform
    // Streaming stores: nothing in this kernel reads these rows again.
    if (a.splits == 1) {
        uint16_t* orow = a.out + (int64_t)it.t * a.out_s0 + (int64_t)head0 * a.out_s1 + 8 * l;
#pragma unroll
        for (int e = 0; e < kRows; ++e) {
            if (e < n_rows) {
                __builtin_nontemporal_store(u32x2{v[e][0], v[e][1]}, (u32x2*)(orow + e * a.out_s1));  // 8-byte aligned rows
                __builtin_nontemporal_store(u32x2{v[e][2], v[e][3]}, (u32x2*)(orow + e * a.out_s1 + 4));
            }
        }
    } else {
        uint16_t* prow = a.ws_o + (((int64_t)it.t * a.splits + it.s) * a.H + head0) * kHeadDim + 8 * l;
#pragma unroll
        for (int e = 0; e < kRows; ++e)
            if (e < n_rows) __builtin_nontemporal_store(v[e], (u32x4*)(prow + e * kHeadDim));
    }
}

// ---------------------------------------------------------------------------
// bf16 KV, narrow layout: one workgroup per (row, block of 16 heads, key
// split).  The four waves are independent: wave w takes the split's 16-key
// tiles w, w+4, w+8, ... through a private two-stage LDS ring, keeps its own
// online softmax and its own O^T for the 16 heads x 512 dims, and the four
// states are merged once, in the epilogue.  The loop has no exchange and no
// barrier: a wave waits only for its own copies.  Products on the 16x16 MFMAs:
//     S^T[16 keys, 16 heads]  = K[keys, d] . Q^T[d, heads]      (16x16x32, 16 k-steps)
//     O^T[16 dims, 16 heads] += K^T[dims, keys] . P^T[keys, heads]   (16x16x16, 32 dim blocks)
// The score output (lane: head l & 15, keys 4*(l >> 4) + i) is already the
// P^T operand layout, so P goes from the softmax straight into the PV MFMA.
// The head blocks of one row are consecutive work items (same XCD) and read
// the same key rows, which L2 then fetches from HBM once.
//
// Tile layout (16 KiB): 1 KiB block kk (the k-step of dims 32kk .. 32kk+31)
// holds at 16-byte position p the chunk 4kk + (p >> 4) (dims 8*chunk .. +8)
// of key row (p & 15) ^ (4*((p >> 4) & 1)).  The score operand of k-step kk
// is then lane l's position (l & 48) | ((l & 15) ^ ((l & 16) >> 2)) of block
// kk, and the transposing PV read of dim block db sits at a per-lane base +
// 512*db; both are conflict-free over every 16 lanes.
// ---------------------------------------------------------------------------
template <bool kDbg>
__global__ __launch_bounds__(256, 1) void attn_narrow_kernel(AttnArgs a) {
    constexpr int kTile = kNarrowTileKeys * 1024;  // 16 KiB
    constexpr int kH = kNarrowHeadsPerBlock;
    __shared__ __attribute__((aligned(1024))) uint8_t s_ring[4][2][kTile];
    __shared__ int32_t s_slot[kNarrowMaxSplitKeys];
    __shared__ int32_t s_table[kTableCap];
    __shared__ float s_ml[4][2][kH];

    fetch_args(a);
    Item it;
    if (!decode_item(a, it)) return;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int head0 = it.hb * kH;

    // Metadata round 1 (request bounds), then Q (independent of it), then
    // the rest of the row resolution.
    const RequestChunk rc = load_requests(a.m, 0, l);
    __builtin_amdgcn_sched_barrier(0);
    // Q^T as the B operand of the score MFMA: lane holds head (l & 15), dims
    // 32*kk + 8*(l >> 4) .. +8 of k-step kk.  Heads past H read head H-1;
    // their results are never written.
    bf16x8 qf[16];
    {
        const uint16_t* qrow =
            a.q + (int64_t)it.t * a.q_s0 + (int64_t)min(head0 + (l & 15), a.H - 1) * a.q_s1 + 8 * (l >> 4);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * kk));
    }
    __builtin_amdgcn_sched_barrier(0);
    const RowKeys rk = row_keys_from(a.m, it.t, l, rc);
    const int k0 = it.s * a.chunk;
    const int n_here = __builtin_amdgcn_readfirstlane(max(0, min(rk.n_swa + rk.n_ext, k0 + a.chunk) - k0));
    build_slots<kNarrowMaxSplitKeys>(a, rk, it.t, k0, n_here, s_slot, s_table, tid);
    // Q and the metadata are retired here, so the only vector-memory
    // operations in flight below are this wave's copies into LDS (16 per
    // tile) and the explicit vmcnt waits count exactly those.
    wait_vmcnt<0>();

    const int n_tiles = (n_here + kNarrowTileKeys - 1) / kNarrowTileKeys;
    const int n_mine = n_tiles > w ? (n_tiles - w + 3) / 4 : 0;  // tiles w, w+4, ...
    const uint32_t ring_w = lds_addr(&s_ring[w][0][0]);

    // Copy of this wave's n-th tile (tile w + 4n) into stage n & 1: lane p
    // moves 16 bytes of row (p & 15) ^ (4*((p >> 4) & 1)) into position p of
    // every block.  Returns the tile's valid-key mask (bit k: key k).
    const int dma_row = (l & 15) ^ (4 * ((l >> 4) & 1));
    auto fetch = [&](int n) -> uint32_t {
        const int key = kNarrowTileKeys * (w + 4 * n) + dma_row;
        const int32_t slot = key < n_here ? s_slot[key] : -1;
        const bool swa = k0 + key < rk.n_swa;
        const uint8_t* row = slot >= 0 ? (swa ? a.swa_pool : a.ext_pool) + (int64_t)slot * (swa ? a.swa_row_bytes : a.ext_row_bytes)
                                       : a.zero_row;
        if constexpr (kDbg) {
            if (l < 16) a.dbg_keys[dbg_unit(a, it) * a.chunk + key] = (uint64_t)(uintptr_t)row;  // dma_row == l
        }
        const uint8_t* src = row + 16 * (l >> 4);
        const uint32_t dst = ring_w + (n & 1) * kTile;
        dma16_off<0>(src, dst);
        dma16_off<64>(src, dst + 1024);
        dma16_off<128>(src, dst + 2048);
        dma16_off<192>(src, dst + 3072);
        dma16_off<256>(src, dst + 4096);
        dma16_off<320>(src, dst + 5120);
        dma16_off<384>(src, dst + 6144);
        dma16_off<448>(src, dst + 7168);
        dma16_off<512>(src, dst + 8192);
        dma16_off<576>(src, dst + 9216);
        dma16_off<640>(src, dst + 10240);
        dma16_off<704>(src, dst + 11264);
        dma16_off<768>(src, dst + 12288);
        dma16_off<832>(src, dst + 13312);
        dma16_off<896>(src, dst + 14336);
        dma16_off<960>(src, dst + 15360);
        return (uint32_t)__ballot(slot >= 0) & 0xFFFFu;  // lanes 0..15 copy rows 0..15
    };

    // Per-lane LDS offsets of the score operand and of the transposing PV
    // read.  PV source lane S = 4k + q of 16-lane block b points at row
    // 4b + k, dims 16*db + 4q .. +3 (chunk 2db + (q >> 1), half q & 1), so
    // result lane 4q + j of the block gets dim 4q + j of rows 4b .. 4b+3.
    const uint32_t s_lane = 16u * ((l & 48) | ((l & 15) ^ ((l & 16) >> 2)));
    const int tq = l & 3, trow = 4 * (l >> 4) + ((l >> 2) & 3), th1 = tq >> 1;
    const uint32_t t_lane = 256u * th1 + 16u * (trow ^ (4 * th1)) + 8u * (tq & 1);

    f32x4 oacc[32];
#pragma unroll
    for (int db = 0; db < 32; ++db) oacc[db] = f32x4{};
    float m_run = -INFINITY, l_part = 0.f;
    const float sl2 = a.scale_log2;
    const int key_shift = 4 * (l >> 4);  // score register i: key 4*(l >> 4) + i

    // Online softmax (base 2).  The running reference m_run (scaled units,
    // per head) is set by the first tile and moves only when a score exceeds
    // it by more than 2^20: probabilities up to 2^20 keep bf16's relative
    // precision and stay far from overflow.  When a head that has already
    // accumulated needs a larger reference, the wave restarts its tiles from
    // the first with that reference (its accumulators are never rescaled, so
    // they stay in place in the accumulation registers); the reference only
    // grows, so restarts are bounded and, for attention scores, rare.
    constexpr float kRefSlackLog2 = 20.0f;
    uint32_t msk0 = 0, msk1 = 0;
    if (n_mine > 0) msk0 = fetch(0);
    if (n_mine > 1) msk1 = fetch(1);
    for (int n = 0; n < n_mine; ++n) {
        if (n + 1 < n_mine) wait_vmcnt<16>();  // tile n landed (tile n+1 may be in flight)
        else wait_vmcnt<0>();
        const uint32_t st = ring_w + (n & 1) * kTile;
        const __attribute__((address_space(3))) uint8_t* sp = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + s_lane);
        const __attribute__((address_space(3))) uint8_t* tp = (const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(st + t_lane);
        // Operand reads in two waves so that at most 48 operand registers are
        // live: the score operand and the first half of the PV operand, then
        // (once the score MFMAs hold their operands) the second half.
        bf16x8 av[16];
        bf16x4 kt[32];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) av[kk] = *(const __attribute__((address_space(3))) bf16x8*)(sp + 1024 * kk);
#pragma unroll
        for (int db = 0; db < 16; ++db) kt[db] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tp + 512 * db));
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sacc = f32x4{};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[kk], qf[kk], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 16; db < 32; ++db) kt[db] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tp + 512 * db));
        const uint32_t msk = (n & 1) ? msk1 : msk0;
        // Every read of this stage has returned: refill it with tile n+2.
        if (n + 2 < n_mine) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const uint32_t nm = fetch(n + 2);
            if (n & 1) msk1 = nm;
            else msk0 = nm;
        }

        // This lane holds keys 4*(l >> 4) .. +3 of head l & 15; the other
        // three quarters of the head's keys sit in lanes l ^ 16, l ^ 32, l ^ 48.
        float sv[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
        if (msk != 0xFFFFu) {
            const uint32_t mine = msk >> key_shift;
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = ((mine >> i) & 1u) ? sv[i] : -INFINITY;
        }
        const float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])) * sl2;
        if (__any(tmax > m_run + kRefSlackLog2)) {
            float hmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            hmax = fmaxf(hmax, __shfl_xor(hmax, 32));  // the head's tile maximum
            const bool grow = hmax > m_run + kRefSlackLog2;
            const bool restart = __any(grow && m_run != -INFINITY);
            m_run = grow ? hmax : m_run;
            if (restart) {
                wait_vmcnt<0>();  // this wave's copies have landed; its stages are free
#pragma unroll
                for (int db = 0; db < 32; ++db) oacc[db] = f32x4{};
                l_part = 0.f;
                msk0 = fetch(0);
                if (n_mine > 1) msk1 = fetch(1);
                n = -1;
                continue;
            }
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        bf16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pr = fast_exp2(fmaf(sv[i], sl2, neg_m));
            l_part += pr;
            pb[i] = (__bf16)pr;
        }
#pragma unroll
        for (int db = 0; db < 32; ++db) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kt[db], pb, oacc[db], 0, 0, 0);
    }

    // Epilogue: merge the four waves' states per head.  M = max of the wave
    // references (and the sink when the row is not split), Z = sum of
    // l_w * 2^(m_w - M) (+ 2^(sink - M)); wave w stages O_w * 2^(m_w - M) / Z
    // as fp32 rows [head][512] in ring quarter w (16-byte chunk c of row h at
    // chunk c ^ h), and wave w then sums the four quarters for heads
    // 4w .. 4w+3 and writes the output (or the normalised partial and its
    // base-2 log-sum-exp for the merge kernel).
    float lh = l_part + __shfl_xor(l_part, 16);
    lh += __shfl_xor(lh, 32);
    __syncthreads();  // every wave is done with the ring
    if (l < kH) {
        s_ml[w][0][l] = lh > 0.f ? m_run : -INFINITY;
        s_ml[w][1][l] = lh;
    }
    __syncthreads();
    const int hd = l & 15;
    const int my_head = head0 + hd;
    float M = (a.splits == 1 && a.sink != nullptr && my_head < a.H) ? a.sink[my_head] * kLog2e : -INFINITY;
    const float sig = M;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, s_ml[v][0][hd]);
    float Z = 0.f, f_own = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float mv = s_ml[v][0][hd];
            Z += mv == -INFINITY ? 0.f : s_ml[v][1][hd] * fast_exp2(mv - M);
        }
        if (sig != -INFINITY) Z += fast_exp2(sig - M);
        const float mw = s_ml[w][0][hd];
        f_own = (mw == -INFINITY || Z <= 0.f) ? 0.f : fast_exp2(mw - M) / Z;
    }
    const float lse2 = Z > 0.f ? M + fast_log2(Z) : -INFINITY;
    {
        uint8_t* q = &s_ring[0][0][0] + w * 32768 + hd * 2048;
#pragma unroll
        for (int db = 0; db < 32; ++db) {
            const int c = 4 * db + (l >> 4);
            const f32x4& o = oacc[db];
            *(f32x4*)(q + 16 * (c ^ hd)) = f32x4{o[0] * f_own, o[1] * f_own, o[2] * f_own, o[3] * f_own};
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h2 = 4 * w + e;
        const int head = head0 + h2;
        if (head >= a.H) break;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint8_t* q = &s_ring[0][0][0] + v * 32768 + h2 * 2048;
            const f32x4 x0 = *(const f32x4*)(q + 16 * ((2 * l) ^ h2));
            const f32x4 x1 = *(const f32x4*)(q + 16 * ((2 * l + 1) ^ h2));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] += x0[i];
                acc[4 + i] += x1[i];
            }
        }
        const u32x4 ov = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                          pack_bf16x2(acc[6], acc[7])};
        const float lse_h = __shfl(lse2, h2);
        if (a.splits == 1) {
            uint16_t* orow = a.out + (int64_t)it.t * a.out_s0 + (int64_t)head * a.out_s1 + 8 * l;
            *(u32x2*)orow = u32x2{ov[0], ov[1]};  // out rows need only 8-byte alignment
            *(u32x2*)(orow + 4) = u32x2{ov[2], ov[3]};
            if (a.lse != nullptr && l == 0) a.lse[(int64_t)it.t * a.lse_s0 + head] = lse_h * kLn2;
        } else {
            const int64_t part = ((int64_t)it.t * a.splits + it.s) * a.H + head;
            *(u32x4*)(a.ws_o + part * kHeadDim + 8 * l) = ov;
            if (l == 0) a.ws_lse[part] = lse_h;
        }
    }
}

// ---------------------------------------------------------------------------
// Packed FP8 KV, two layouts (kHH = head groups of 32 per workgroup):
//  - kHH = 2: 64-head workgroups, wave (hh, dq) owning heads 32hh .. +31 and
//    dims 256dq .. +255 of both products; the two dim halves of a head group
//    add their score partials;
//  - kHH = 1: 32-head workgroups, wave dq owning all 32 heads and dims
//    128dq .. +127; the four dim quarters add their score partials.  Half the
//    products and operand decodes per wave and tile, for batches whose
//    64-head grid leaves compute units idle.  The raw records stream into a
// 4-stage LDS ring with direct global->LDS copies, three tiles ahead, and
// both MFMA operands are decoded straight from the ring into registers:
//  - S^T = K.Q^T: lane l reads 8 codes of key l & 31 (one 8-byte read per
//    k-step) and converts them to bf16 with gfx950's conversion instruction
//    (exact: every E4M3 value is a bf16 value); rotary k-steps read bf16;
//  - O^T += K^T.P^T: the transposing 8-bit LDS read gives each lane one dim
//    of 8 keys (16 lanes read 8 keys x 16 dims: source lane s of a 16-lane
//    group addresses the key that P^T holds as element s / 2, at dims
//    (first dim + 8 (s % 2)), and lane i receives dim (first dim + i) of the
//    8 keys, in element order); rotary dims use the 16-bit transposing read
//    (source lane s: element s / 4, dims (first dim + 4 (s % 4)); a second
//    read 8 keys on gives elements 4..7).  P^T's element e of lane half h
//    in k-step pp is tile key 16 pp + 4 h + (e % 4) + 8 (e / 4), the order
//    of the score tile's MFMA output rows.
// (The descriptions below use the 64-head layout's 256-dim slices; the
// 32-head layout's 128-dim slices are the same with 128 in place of 256.)
// The per-token scale multiplies the fp32 non-rotary score partial and is
// folded into P for the non-rotary PV product, so the decode adds no
// rounding.  Two barriers per tile: one when the tile has landed, one in
// the score exchange.
//
// A split walks its row's compressed entries first, then the window
// (prefetch_slots / finish_slots), so that its first loads need nothing
// from the row's request bounds.
//
// Ring stage: record of tile key k (its 576 bytes as stored: 448 codes, 64
// bf16 rotary dims) at byte 592 k (a 16-byte pad after each record spreads
// the keys of a read over the LDS banks); wave w copies keys 8w .. 8w+7 and
// their scales (into a separate 128-byte slot per stage).
// ---------------------------------------------------------------------------
constexpr int kFp8Stages = 4;
constexpr int kFp8RecSlot = 592;                       // LDS bytes per record (36 chunks + 1 pad chunk)
constexpr int kFp8RawStage = kTileKeys * kFp8RecSlot;  // 18944
constexpr int kFp8CopiesPerTile = 6;                   // per wave: 5 record copies + 1 scale copy

// Direct global -> LDS copy of 4 bytes per lane: lane i's bytes land at LDS
// byte address lds_base + 4*i (see dma16_off).
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base)
        : "memory");
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Eight E4M3 codes (two words) -> eight bf16, in order.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(bf16x8, u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                            e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)});
}

template <int kHH, bool kDbg>
__global__ __launch_bounds__(256, 1) void attn_fp8_kernel(AttnArgs a) {
    constexpr int kDims = 128 * kHH;   // head dims per wave (a dim slice)
    constexpr int kSteps = kDims / 16;  // score k-steps per wave and tile
    constexpr int kMb = kDims / 32;     // PV dim blocks per wave
    constexpr int kHeads = 32 * kHH;    // heads per workgroup
    static_assert(kHH == 1 || kHH == 2, "one or two 32-head groups");
    __shared__ __attribute__((aligned(1024))) uint8_t s_raw[kFp8Stages][kFp8RawStage];
    __shared__ __attribute__((aligned(16))) float s_rsc[kFp8Stages][kTileKeys];
    __shared__ __attribute__((aligned(16))) float s_sx[4 * 64 * 16];
    __shared__ int32_t s_slot[kMaxSplitKeys];
    // The page-table cache is needed only while the slot list is built, before
    // the exchange buffer's first use.
    int32_t* const s_table = (int32_t*)s_sx;
    static_assert(kTableCap * 4 <= sizeof(s_sx), "page-table cache fits the exchange buffer");
    static_assert(2 * 32 * 1024 <= sizeof(s_raw), "the ring holds the epilogue's two 32-head staging blocks");

    fetch_args(a);
    Item it;
    if (!decode_item(a, it)) return;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int hh = kHH == 2 ? w >> 1 : 0;  // head group
    const int dq = kHH == 2 ? w & 1 : w;   // dim slice

    // The request bounds first (the first wait, for them, leaves every later
    // load in flight), then the slot list's loads that do not need them,
    // then Q^T as the B operand of the scores (lane: head 32hh + (l & 31),
    // dims kDims*dq + 16j + 8(l >> 5) .. +8 of k-step j; heads past H read
    // head H-1, whose results are never written).
    const RequestChunk rc = load_requests(a.m, 0, l);
    const int k0 = it.s * a.chunk;
    SlotPrefetch pf;
    prefetch_slots(a, it.t, k0, tid, pf);
    bf16x8 qf[kSteps];
    {
        const int head = min(it.hb * kHeads + 32 * hh + (l & 31), a.H - 1);
        const uint16_t* qrow = a.q + (int64_t)it.t * a.q_s0 + (int64_t)head * a.q_s1 + kDims * dq + 8 * (l >> 5);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) qf[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * j));
    }

    const RowKeys rk = row_keys_from(a.m, it.t, l, rc);
    const int n_here = max(0, min(rk.n_swa + rk.n_ext, k0 + a.chunk) - k0);
    const int n_tiles = (n_here + kTileKeys - 1) / kTileKeys;
    finish_slots(a, rk, k0, n_here, pf, s_slot, s_table, tid);

    // Copies of tile j into stage j % 4: five 16-byte copies per lane over
    // the wave's 8 x 37 record slots (slot f = 64 i + l is chunk f % 37 of
    // key 8w + f / 37, chunk 36 being the pad, filled from the zero row; the
    // last copy has 40 lanes), and one 4-byte copy of the 8 scales (lanes
    // 0..7).  Lane k < 32 resolves the record and scale addresses of tile key
    // k; each copying lane fetches its key's addresses with a cross-lane
    // permute.  Unused keys read the zero row (codes, rotary dims and scale
    // all zero).
    int src_lane[5], chunk_off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int f = 64 * i + l;
        const int e = min(f / 37, 7);
        src_lane[i] = 4 * (8 * w + e);
        chunk_off[i] = f - 37 * (f / 37);  // 36: the pad
    }
    auto bperm64 = [](int src4, uint64_t v) -> uint64_t {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)(uint32_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)(uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | lo;
    };
    // Returns the tile's mask of used keys (bit k: tile key k).
    auto issue_tile = [&](int j) -> uint64_t {
        const int tb = j * kTileKeys;
        uint64_t rec_ad, sc_ad;
        bool used;
        {
            const int key = tb + (l & 31);
            const int32_t slot = key < n_here ? s_slot[key] : -1;
            used = l < 32 && slot >= 0;
            const uint8_t* page = (k0 + key < rk.n_ext ? a.ext_pool : a.swa_pool) + (int64_t)(slot >> 8) * kFp8PageBytes;
            rec_ad = (uint64_t)(uintptr_t)(slot >= 0 ? page + (slot & 255) * kFp8RecBytes : a.zero_row);
            sc_ad = (uint64_t)(uintptr_t)(slot >= 0 ? page + kFp8ScaleOffset + 4 * (slot & 255) : a.zero_row);
        }
        if constexpr (kDbg) {
            if (l < 32) a.dbg_keys[dbg_unit(a, it) * a.chunk + tb + l] = rec_ad;
        }
        const uint32_t dst = lds_addr(&s_raw[j % kFp8Stages][8 * w * kFp8RecSlot]);
        // Every permute before the first copy (the copies are ordered asm, so
        // alternating the two would wait out each permute on its own).
        uint64_t row[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) row[i] = bperm64(src_lane[i], rec_ad);
        const uint64_t scp = bperm64(4 * (8 * w + (l & 7)), sc_ad);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint8_t* src = chunk_off[i] < 36 ? (const uint8_t*)(uintptr_t)row[i] + 16 * chunk_off[i] : a.zero_row;
            if (i < 4 || l < 8 * 37 - 256) dma16_off<0>(src, dst + 1024 * i);
        }
        if (l < 8) dma4((const void*)(uintptr_t)scp, lds_addr(&s_rsc[j % kFp8Stages][8 * w]));
        return __ballot(used);
    };

    f32x16 oacc[kMb];
#pragma unroll
    for (int mb = 0; mb < kMb; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // Q and the slot list have arrived (the compiler waited for the window
    // page entries, issued after Q); the explicit wait tells it so before
    // any copy.
    wait_vmcnt<0>();
    // Used-key masks of the tiles in flight (tiles j, j+1, j+2).
    uint64_t vm0 = n_tiles > 0 ? issue_tile(0) : 0;
    uint64_t vm1 = n_tiles > 1 ? issue_tile(1) : 0;
    uint64_t vm2 = n_tiles > 2 ? issue_tile(2) : 0;
    static_assert(kFp8Stages == 4, "three tiles in flight");

    // Per-lane constants of the operand reads.
    const int key_s = l & 31;                      // score operand: this lane's key
    const int g = l >> 4, gi = l & 15;             // transposing reads: 16-lane group, lane in it
    // One instance of the loop per dim slice (kD = dq): a branch on dq inside
    // the loop made the compiler copy all the accumulators on every tile.
    auto tile_loop = [&](auto d_tag) __attribute__((always_inline)) {
        for (int j = 0; j < n_tiles; ++j) {
            // This wave's copies of tile j (those of j+1 and j+2 may still be in
            // flight); then every wave's.
            if (j + 2 < n_tiles) wait_vmcnt<2 * kFp8CopiesPerTile>();
            else if (j + 1 < n_tiles) wait_vmcnt<kFp8CopiesPerTile>();
            else wait_vmcnt<0>();
            __syncthreads();  // tile j in LDS for every wave; every wave is done with tile j-1's stage
            // Stage (j+3) % 4 held tile j-1.
            const uint64_t vmask = vm0;
            vm0 = vm1;
            vm1 = vm2;
            vm2 = j + kFp8Stages - 1 < n_tiles ? issue_tile(j + kFp8Stages - 1) : 0;
            const uint8_t* stage = &s_raw[j % kFp8Stages][0];

            // S^T partial over this wave's kDims dims: the non-rotary k-steps
            // (dims < 448) and the rotary ones (the last slice's last four
            // k-steps) accumulate apart; the non-rotary partial is scaled per
            // key.  The dim slices are separate instances (kD), so that every
            // operand is a fixed register.
            f32x16 sacc = f32x16{};
            float sc_key[16];
            auto scores = [&](auto d_tag) __attribute__((always_inline)) {
                constexpr int kD = decltype(d_tag)::value;
                constexpr int kLo = kDims * kD;  // the slice's first dim (every slice starts below 448)
                constexpr int kNopeSteps = (kNope - kLo) / 16 < kSteps ? (kNope - kLo) / 16 : kSteps;
                static_assert(kLo < kNope && (kNope - kLo) % 16 == 0, "slices start at non-rotary dims");
                const uint8_t* rec = stage + key_s * kFp8RecSlot + kLo + 8 * (l >> 5);
                u32x2 cn[kNopeSteps];
                u32x4 cr[kSteps - kNopeSteps + 1];
    #pragma unroll
                for (int jj = 0; jj < kNopeSteps; ++jj) cn[jj] = *(const u32x2*)(rec + 16 * jj);
    #pragma unroll
                for (int q = 0; q < kSteps - kNopeSteps; ++q) {  // bf16 dims 448 + 16q + 8(l >> 5) .. +8
                    cr[q] = *(const u32x4*)(stage + key_s * kFp8RecSlot + kNope + 32 * q + 16 * (l >> 5));
                }
                // Every read in flight before the first product (left alone, the
                // scheduler issues one read ahead of its use, and with one wave
                // per SIMD nothing hides the LDS latency of each).
                __builtin_amdgcn_sched_barrier(0);
                f32x16 sacc_r = f32x16{};
    #pragma unroll
                for (int jj = 0; jj < kNopeSteps; ++jj)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16x8(cn[jj][0], cn[jj][1]), qf[jj], sacc, 0, 0, 0);
    #pragma unroll
                for (int q = 0; q < kSteps - kNopeSteps; ++q)
                    sacc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cr[q]), qf[kNopeSteps + q], sacc_r, 0, 0, 0);
    #pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4 sc4 = *(const f32x4*)(&s_rsc[j % kFp8Stages][8 * qd + 4 * (l >> 5)]);
    #pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        sc_key[4 * qd + jj] = sc4[jj];
                        sacc[4 * qd + jj] = sacc[4 * qd + jj] * sc4[jj] + sacc_r[4 * qd + jj];
                    }
                }
            };
            scores(d_tag);
            if constexpr (kHH == 2) exchange_partial(s_sx, w, l, sacc);
            else exchange_partial4(s_sx, w, l, sacc);

            bf16x8 pb[2], pbs[2];
            softmax_tile<true>(sacc, vmask, a.scale_log2, l, sc_key, m_run, l_run, oacc, pb, pbs);

            // O^T += K^T . P^T: lane l holds dim kDims*dq + 32mb + (l & 31) of the
            // eight keys 16pp + 4h + {0..3, 8..11}, h = l >> 5, in the order in
            // which P^T holds them (the score tile's MFMA output layout: lane
            // half h holds keys 8q + 4h + {0..3} in registers 4q .. 4q+3); the
            // transposing reads' source lanes address those keys.
            // All operand reads go out before the products.
            auto pv = [&](auto d_tag) __attribute__((always_inline)) {
                constexpr int kD = decltype(d_tag)::value;
                constexpr int kLo = kDims * kD;
                constexpr int kNopeMb = (kNope - kLo) / 32 < kMb ? (kNope - kLo) / 32 : kMb;  // dim blocks below 448
                static_assert((kNope - kLo) % 32 == 0, "dim blocks do not straddle the rotary boundary");
                i32x2 c8[2 * kNopeMb];
                bf16x4 c16[2 * (kMb - kNopeMb) + 1][2];  // (+1: no zero-length array for an all-FP8 slice)
    #pragma unroll
                for (int mb = 0; mb < kNopeMb; ++mb)
    #pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int dim_base = kLo + 32 * mb + 16 * (g & 1);
                        const int js = gi >> 1;  // the key this source lane addresses: element js of the operand
                        const int key = 16 * pp + 4 * (g >> 1) + (js & 3) + 8 * (js >> 2);
                        const uint8_t* p0 = stage + key * kFp8RecSlot + dim_base + 8 * (gi & 1);
                        c8[2 * mb + pp] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)lds_addr(p0));
                    }
    #pragma unroll
                for (int mb = kNopeMb; mb < kMb; ++mb)
    #pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int dim_base = kLo + 32 * mb + 16 * (g & 1);
                        const int key = 16 * pp + 4 * (g >> 1) + (gi >> 2);  // elements 0..3; 4..7 are 8 keys on
                        const uint8_t* p0 = stage + key * kFp8RecSlot + kNope + 2 * (dim_base - kNope + 4 * (gi & 3));
                        c16[2 * (mb - kNopeMb) + pp][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)lds_addr(p0));
                        c16[2 * (mb - kNopeMb) + pp][1] =
                            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)lds_addr(p0 + 8 * kFp8RecSlot));
                    }
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int mb = 0; mb < kNopeMb; ++mb)
    #pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
                        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            e4m3x8_to_bf16x8((uint32_t)c8[2 * mb + pp][0], (uint32_t)c8[2 * mb + pp][1]), pbs[pp], oacc[mb], 0, 0, 0);
    #pragma unroll
                for (int mb = kNopeMb; mb < kMb; ++mb)
    #pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const bf16x4 lo = c16[2 * (mb - kNopeMb) + pp][0], hi = c16[2 * (mb - kNopeMb) + pp][1];
                        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]},
                                                                          pb[pp], oacc[mb], 0, 0, 0);
                    }
            };
            pv(d_tag);
        }
    };
    if (dq == 0) tile_loop(std::integral_constant<int, 0>{});
    else if (dq == 1) tile_loop(std::integral_constant<int, 1>{});
    else if constexpr (kHH == 1) {
        if (dq == 2) tile_loop(std::integral_constant<int, 2>{});
        else tile_loop(std::integral_constant<int, 3>{});
    }
    write_result<kHH>(a, it, hh, dq, l, oacc, m_run, l_run, &s_raw[0][0], &s_raw[0][0] + 32 * 1024);
}

// ---------------------------------------------------------------------------
// Merge of split partials + sink: one wave per (row, head), 8 dims per lane;
// every split's lse and partial row are loaded before any is combined, so a
// row's merge costs one round of loads.
// ---------------------------------------------------------------------------
// kPass: splits per pass (the smallest of 2, 4, 8, 16 that covers the
// splits, so no load is wasted on a clamped duplicate; only kPass = 16 loops,
// over more than 16 splits).
template <int kPass>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
    // Every kernel argument used below, in one round of scalar loads.
    asm volatile("" ::"s"(a.H), "s"(a.splits), "s"(a.ws_lse), "s"(a.ws_o), "s"(a.sink), "s"(a.zero_row), "s"(a.out),
                 "s"(a.out_s0), "s"(a.out_s1), "s"(a.lse), "s"(a.lse_s0));
    // Work item (row t, heads 4q .. 4q+3) of workgroup b, laid out like the
    // split kernels' items (decode_item): XCD b & 7 takes a contiguous run of
    // items, so a row's merge runs on the XCD that wrote its partials.
    const int n_quads = (a.H + 3) >> 2;
    const int n = a.T * n_quads;
    const int per_xcd = (n + 7) >> 3;
    const int slot = blockIdx.x >> 3;
    const int raw = (blockIdx.x & 7) * per_xcd + slot;
    if (slot >= per_xcd || raw >= n) return;
    const int t = raw / n_quads;
    const int head = (raw - t * n_quads) * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (head >= a.H) return;
    const int S = a.splits;
    const float* lp = a.ws_lse + (int64_t)t * S * a.H + head;
    const uint16_t* ob = a.ws_o + ((int64_t)t * S * a.H + head) * kHeadDim + 8 * l;
    const int64_t ostride = (int64_t)a.H * kHeadDim;
    // The sink is read from a valid address either way (the zero row when
    // there is none) so that its load does not hold up the others.
    const float sink_raw = a.sink != nullptr ? a.sink[head] : *(const float*)a.zero_row;
    const float sig = a.sink != nullptr ? sink_raw * kLog2e : -INFINITY;
    // Running base-2 merge of the splits; the sink joins at the end.
    float M = -INFINITY, Z = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto pass = [&](int k0) {
        // Every load of the pass is issued before any is used, with split
        // indices clamped into range (a clamped duplicate gets weight zero),
        // so a pass costs one memory round trip.  An empty split left its
        // partial stale: its weight is zero and the select below drops it.
        u32x4 x[kPass];
#pragma unroll
        for (int j = 0; j < kPass; ++j) x[j] = *(const u32x4*)(ob + min(k0 + j, S - 1) * ostride);
        const float lse_l = lp[(int64_t)min(k0 + (l & (kPass - 1)), S - 1) * a.H];
        float lv[kPass];
        float pm = -INFINITY;
#pragma unroll
        for (int j = 0; j < kPass; ++j) {
            lv[j] = k0 + j < S ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lse_l), j))
                               : -INFINITY;
            pm = fmaxf(pm, lv[j]);
        }
        const float Mn = fmaxf(M, pm);
        if (Mn == -INFINITY) return;  // nothing seen yet
        const float r = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
        Z *= r;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= r;
        M = Mn;
#pragma unroll
        for (int j = 0; j < kPass; ++j) {
            const float w = lv[j] == -INFINITY ? 0.f : fast_exp2(lv[j] - M);
            Z += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __builtin_bit_cast(float, x[j][e] << 16);
                const float hi = __builtin_bit_cast(float, x[j][e] & 0xFFFF0000u);
                acc[2 * e] += w != 0.f ? w * lo : 0.f;
                acc[2 * e + 1] += w != 0.f ? w * hi : 0.f;
            }
        }
    };
    if constexpr (kPass < 16) {
        pass(0);  // the launcher picks kPass >= splits: one round trip, no loop
    } else {
        for (int k0 = 0; k0 < S; k0 += kPass) pass(k0);
    }
    // The sink: one more logit with value zero.
    const float Mf = fmaxf(M, sig);
    if (Mf != -INFINITY) {
        const float r = M == -INFINITY ? 0.f : fast_exp2(M - Mf);
        Z = Z * r + fast_exp2(sig - Mf);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= r;
    }
    M = Mf;
    const float f = Z > 0.f ? 1.f / Z : 0.f;
    uint16_t* orow = a.out + (int64_t)t * a.out_s0 + (int64_t)head * a.out_s1 + 8 * l;
    u32x4 v = {pack_bf16x2(acc[0] * f, acc[1] * f), pack_bf16x2(acc[2] * f, acc[3] * f),
               pack_bf16x2(acc[4] * f, acc[5] * f), pack_bf16x2(acc[6] * f, acc[7] * f)};
    *(u32x4*)orow = v;
    if (a.lse != nullptr && l == 0)
        a.lse[(int64_t)t * a.lse_s0 + head] = (M == -INFINITY) ? -INFINITY : (M + fast_log2(Z)) * kLn2;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <bool kDbg>
void launch_split(const AttnArgs& a, Layout layout, dim3 grid, hipStream_t stream) {
    switch (layout) {
        case Layout::kFp8:
            hipLaunchKernelGGL(HIP_KERNEL_NAME(attn_fp8_kernel<2, kDbg>), grid, dim3(256), 0, stream, a);
            break;
        case Layout::kFp8H32:
            hipLaunchKernelGGL(HIP_KERNEL_NAME(attn_fp8_kernel<1, kDbg>), grid, dim3(256), 0, stream, a);
            break;
        case Layout::kWide:
            hipLaunchKernelGGL((attn_wide_kernel<2, kDbg>), grid, dim3(256), 0, stream, a);
            break;
        case Layout::kWide32:
            hipLaunchKernelGGL((attn_wide_kernel<1, kDbg>), grid, dim3(256), 0, stream, a);
            break;
        case Layout::kRoles32:
            hipLaunchKernelGGL((attn_ws_kernel<1, kDbg>), grid, dim3(256), 0, stream, a);
            break;
        case Layout::kNarrow:
            hipLaunchKernelGGL(attn_narrow_kernel<kDbg>, grid, dim3(256), 0, stream, a);
            break;
    }
}

hipError_t launch_attention(const AttnArgs& a, Layout layout, hipStream_t stream) {
    const int per_xcd = (a.n_items + 7) / 8;
    const dim3 grid((unsigned)(8 * per_xcd));
    if (a.dbg_keys != nullptr)
        launch_split<true>(a, layout, grid, stream);
    else
        launch_split<false>(a, layout, grid, stream);
    return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, hipStream_t stream) {
    const int64_t n = (int64_t)a.T * ((a.H + 3) / 4);  // (row, 4 heads) items; 8 XCDs x ceil(n / 8) workgroups
    const dim3 grid((unsigned)(8 * ((n + 7) / 8)));
    if (a.splits <= 2)
        hipLaunchKernelGGL(merge_kernel<2>, grid, dim3(256), 0, stream, a);
    else if (a.splits <= 4)
        hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(256), 0, stream, a);
    else if (a.splits <= 8)
        hipLaunchKernelGGL(merge_kernel<8>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(merge_kernel<16>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& g, hipStream_t stream) {
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)g.T), dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace dsv4
