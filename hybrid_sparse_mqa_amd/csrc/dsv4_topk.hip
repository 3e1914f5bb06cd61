// dsv4_topk.hip -- C4 top-k selection: for every query row, the K candidate
// compressed entries with the highest indexer scores (the DeepSeek-V4 /
// SGLang overview page: the indexer keeps the top 512 compressed entries per
// query, its kernel section naming a Lightning TopK kernel that replaces a
// global sort by a radix select), produced as the c4_indices the attention
// reads.  Equal scores: the lower index wins, and -0.0 equals +0.0.  Output:
// the kept indices in ascending order, then -1.
//
// The selection is a radix select on 32-bit keys that order like the scores.
// The first digit (the top 12 key bits) splits the candidates into those
// above the threshold digit D0 (all kept) and those at it; among the latter
// the `need` best (key descending, then index ascending) are kept: directly
// by rank when they are few, else by two more 10-bit key digits and, for
// candidates equal to the threshold key, a radix select on their indices.
// Every kept index's output position is its rank among the kept indices.
//
// Short rows (ld < kTopkSplitMin): one workgroup per row does everything
// (the candidates at D0 -- usually a few dozen -- move to LDS).
//
// Long rows (the C4 entries of long contexts, e.g. 2^18 at 1M tokens) read
// the scores from HBM once, with many workgroups per row:
//   topk_chunk_kernel   one workgroup per 16384-candidate chunk: the chunk's
//                       own first-digit histogram (LDS) and threshold (the
//                       largest digit d with count(digit >= d) >= K), and the
//                       (key, index) of every candidate at or above it
//                       appended to the row's survivor list.  Every
//                       candidate of the row's top K is in its chunk's top K,
//                       so the list holds the whole answer.  Each full chunk
//                       also offers a lower bound on the row's threshold
//                       digit: with C full chunks and q = ceil(K / C), the
//                       largest digit d_c with count(digit >= d_c) >= q in
//                       chunk c; min_c d_c has at least C q >= K candidates
//                       at or above it, so the row's K-th best lies there too;
//   topk_finish_kernel  one workgroup per row: the list entries at or above
//                       that bound (usually a tenth of the list) are
//                       compacted into LDS and selected there (first-digit
//                       histogram, split, selection at the threshold); a
//                       list with too many of them takes the general route:
//                       the fine first digit's histogram over the whole list,
//                       then a second pass moves the candidates above D0 to
//                       the kept list and those at it to LDS.  It also clears
//                       the row's counters for the next call.  A row whose
//                       list overflowed its capacity, or whose threshold
//                       digit holds too many candidates for LDS (heavy ties),
//                       runs the selection over the whole row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "dsv4_launch.h"

namespace dsv4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;
constexpr int kBins = kTopkBins;  // digits of 12, 10 and 10 bits
constexpr int kCompCap = 4096;    // candidates at the threshold digit kept in LDS
constexpr int kRankMax = 256;     // candidates at the threshold digit chosen by direct ranking
constexpr int kFineBits = 14;     // first digit of the finishing workgroup (top key bits)
constexpr int kFineBins = 1 << kFineBits;
constexpr int kBitmapMax = 1 << 18;  // candidate ranges ordered through an LDS bitmap
constexpr int kShift[3] = {20, 10, 0}, kNb[3] = {4096, 1024, 1024};

// Order-preserving key: a > b as scores (with -0 == +0) iff key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x + 0.0f);  // -0.0 + 0.0 = +0.0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS of one selecting workgroup.  sel holds the kept indices (padded to a
// multiple of 16 with INT32_MAX for the rank sort); ckey / cidx the
// candidates at the threshold digit (padded likewise for the ranking).
struct Smem {
    __attribute__((aligned(16))) uint32_t hist[kFineBins];  // 4096 bins for the radix passes, 16384 for the fine first digit
    uint32_t pick[2];
    uint32_t wsum[4];
    uint32_t count;
    uint32_t kmax;
    uint32_t trash[3][kThreads];  // per-lane targets of the stores of elements not taken
    __attribute__((aligned(16))) int32_t sel[kTopkMaxK + 16];
    __attribute__((aligned(16))) uint32_t ckey[kCompCap + 16];
    __attribute__((aligned(16))) int32_t cidx[kCompCap + 16];
};
// The output bitmap (once selected) lives in hist: word w of the bitmap at
// word 36 (w / 32) + w % 32, so that the 32 words each thread scans start
// 144 bytes apart and 16 lanes' 16-byte reads hit 16 different bank groups.
__device__ __forceinline__ int bitmap_word(int w) { return 36 * (w >> 5) + (w & 31); }
static_assert(36 * (kBitmapMax / 32 / 32) + 20 * 256 <= kFineBins, "the bitmap and its word places fit the histogram's place");
static_assert(kBins + 2 * kCompCap <= kFineBins, "the bounded entries fit above the first digit's bins");

// Adds one to hist[bin] for the active lanes; the lanes that share the first
// active lane's bin add with one atomic.  For passes over whole rows, where
// ties or a narrow score range would serialise thousands of lanes on one
// LDS address; bounded passes use plain atomics.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int first = __builtin_ctzll(act);
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
    const uint64_t same = __ballot(active && bin == b0);
    if (active && bin != b0) atomicAdd(&hist[bin], 1u);
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], (uint32_t)__popcll(same));
}

// Exclusive prefix of `v` over the lanes of the wave, and the wave's total.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t& total) {
    const int l = threadIdx.x & 63;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t up = __shfl_up(incl, o);
        if (l >= o) incl += up;
    }
    total = __shfl(incl, 63);
    return incl - v;
}

// Exclusive prefix of `v` over the workgroup of kT threads, and its total
// (every thread must call it; `wsum` is kT / 64 words of LDS).
template <int kT = kThreads>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t& total, uint32_t* wsum) {
    const int w = threadIdx.x >> 6;
    uint32_t wt;
    const uint32_t ex = wave_scan(v, wt);
    __syncthreads();  // the previous use of wsum is over
    if ((threadIdx.x & 63) == 0) wsum[w] = wt;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int u = 0; u < kT / 64; ++u) {
        const uint32_t x = wsum[u];
        before += u < w ? x : 0u;
        total += x;
    }
    return before + ex;
}

// The digit of one radix pass from the LDS histogram hist[0 .. kNbT), by all
// kT threads of the workgroup (each holds kNbT/kT consecutive bins).
// Descending (top keys): the largest d with count(digit >= d) >= need;
// out[1] = count(digit > d).  Ascending (low indices): the smallest d with
// count(digit <= d) >= need; out[1] = count(digit < d).  out[0] = d.
// need >= 1 and the histogram total >= need; exactly one thread writes out.
// The caller synchronises before reading out.
template <bool kDescending, int kNbT, int kT = kThreads>
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t need, uint32_t* out, uint32_t* wsum) {
    constexpr int kPerT = kNbT / kT;
    static_assert(kPerT * kT == kNbT && kPerT % 4 == 0, "whole 16-byte groups of bins per thread");
    const int tid = threadIdx.x;
    uint32_t v[kPerT];
#pragma unroll
    for (int j = 0; j < kPerT; j += 4) {
        const uint4 q = *(const uint4*)(hist + kPerT * tid + j);
        v[j] = q.x;
        v[j + 1] = q.y;
        v[j + 2] = q.z;
        v[j + 3] = q.w;
    }
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kPerT; ++j) mine += v[j];
    uint32_t total;
    uint32_t le = block_scan<kT>(mine, total, wsum);  // count(digit < kPerT*tid)
    // Branch-free search of this thread's bins; one store by the one thread
    // whose bins hold the digit.
    int found = -1;
    uint32_t skip = 0;
#pragma unroll
    for (int j = 0; j < kPerT; ++j) {
        const uint32_t lt = le;  // count(digit < d), d = kPerT*tid + j
        le += v[j];              // count(digit <= d)
        const bool hit = kDescending ? (total - lt >= need && total - le < need)  // count(>= d) >= need > count(>= d+1)
                                     : (le >= need && lt < need);                // count(<= d) >= need > count(<= d-1)
        found = hit ? j : found;
        skip = hit ? (kDescending ? total - le : lt) : skip;
    }
    if (found >= 0) {
        out[0] = (uint32_t)(kPerT * tid + found);
        out[1] = skip;
    }
}

// One radix pass: the histogram of digit (v >> shift) & (nb-1) over the
// elements e < n for which `match` holds (v = key_of(e)), then the pick.
// Leaves the digit in pick[0], the skipped count in pick[1] and the chosen
// bin's count in *n_bin (for every thread).
template <bool kDescending, int nb, typename KeyOf, typename Match>
__device__ __forceinline__ void radix_pass(Smem& s, int n, int shift, uint32_t need, KeyOf key_of, Match match,
                                           uint32_t* n_bin) {
    const int tid = threadIdx.x;
    const bool plain = n <= kCompCap;  // few elements: plain atomics (bounded serialisation)
    for (int j = tid; j < nb; j += kThreads) s.hist[j] = 0;
    __syncthreads();
    // kUnroll elements per thread per step, all loaded before any is used
    // (one load round trip per step, not per element); a uniform trip count,
    // so every lane reaches the ballots.
    for (int c0 = 0; c0 < n; c0 += kThreads * kUnroll) {
        uint32_t v[kUnroll];
        bool m[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int c = c0 + tid + kThreads * j;
            v[j] = key_of(min(c, n - 1));
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int c = c0 + tid + kThreads * j;
            m[j] = c < n && match(min(c, n - 1), v[j]);
        }
        if (plain) {
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                if (m[j]) atomicAdd(&s.hist[(v[j] >> shift) & (uint32_t)(nb - 1)], 1u);
        } else {
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) hist_add(s.hist, (v[j] >> shift) & (uint32_t)(nb - 1), m[j]);
        }
    }
    __syncthreads();
    pick_digit<kDescending, nb>(s.hist, need, s.pick, s.wsum);
    __syncthreads();
    *n_bin = s.hist[s.pick[0]];
    __syncthreads();  // hist and pick are reused by the next pass
}

// Digits 2 and 3 and the index tie-break among the m elements whose top
// digit is d0 (others may be present; they do not match): returns, in
// prefix / last, the rule "kept iff key > prefix, or key == prefix and
// index < last" that keeps exactly `need` of them.
template <typename KeyOf, typename IdxOf>
__device__ __forceinline__ void later_digits(Smem& s, int m, uint32_t d0, uint32_t need, KeyOf key_of, IdxOf idx_of,
                                             uint32_t& prefix, int32_t& last) {
    prefix = d0 << kShift[0];
    uint32_t pmask = 0xFFF00000u, n_at = 0;
    for (int p = 1; p < 3; ++p) {  // digits of 10 bits
        const uint32_t pm = pmask, pf = prefix;
        radix_pass<true, 1024>(s, m, kShift[p], need, key_of, [=](int, uint32_t v) { return (v & pm) == pf; },
                               &n_at);
        need -= s.pick[1];
        prefix |= s.pick[0] << kShift[p];
        pmask |= (uint32_t)(kNb[p] - 1) << kShift[p];
    }
    last = INT32_MAX;  // keep equal keys with index < last
    if (need < n_at) {
        uint32_t ip = 0, imask = 0, ineed = need, n_in = 0;
        const uint32_t T = prefix;
        for (int p = 0; p < 3; ++p) {
            const uint32_t im = imask, ipf = ip;
            auto idx_key = [&](int e) { return (uint32_t)idx_of(e); };
            auto tied = [&, T, im, ipf](int e, uint32_t v) { return key_of(e) == T && (v & im) == ipf; };
            if (p == 0)
                radix_pass<false, 4096>(s, m, kShift[p], ineed, idx_key, tied, &n_in);
            else
                radix_pass<false, 1024>(s, m, kShift[p], ineed, idx_key, tied, &n_in);
            ineed -= s.pick[1];
            ip |= s.pick[0] << kShift[p];
            imask |= (uint32_t)(kNb[p] - 1) << kShift[p];
        }
        last = (int32_t)ip + 1;  // the need-th equal key is at index ip
    }
}

// Keeps the `need` best (key descending, then index ascending) of the m
// candidates at threshold digit d0 (the top kDigitBits >= 12 key bits) held
// in s.ckey / s.cidx, appending their indices to s.sel from s.count on.
template <int kDigitBits = 12>
__device__ __forceinline__ void select_at_threshold(Smem& s, int m, uint32_t d0, uint32_t need) {
    const int tid = threadIdx.x;
    const uint32_t base = s.count;
    if (m <= kRankMax) {
        // Direct ranking: candidate e is kept iff fewer than `need`
        // candidates beat it; its rank is then its place.  The list is read
        // 16 bytes at a time, 4 reads in flight (the tail past m is padded
        // with keys that beat nothing).
        const int m16 = (m + 15) & ~15;
        for (int f = m + tid; f < m16; f += kThreads) {
            s.ckey[f] = 0u;
            s.cidx[f] = INT32_MAX;
        }
        __syncthreads();
        for (int e = tid; e < m; e += kThreads) {
            const uint32_t ke = s.ckey[e];
            const int32_t ie = s.cidx[e];
            uint32_t r = 0;
            for (int f = 0; f < m16; f += 16) {
                uint4 kq[4];
                int4 iq[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    kq[u] = *(const uint4*)&s.ckey[f + 4 * u];
                    iq[u] = *(const int4*)&s.cidx[f + 4 * u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    r += (kq[u].x > ke || (kq[u].x == ke && iq[u].x < ie)) ? 1u : 0u;
                    r += (kq[u].y > ke || (kq[u].y == ke && iq[u].y < ie)) ? 1u : 0u;
                    r += (kq[u].z > ke || (kq[u].z == ke && iq[u].z < ie)) ? 1u : 0u;
                    r += (kq[u].w > ke || (kq[u].w == ke && iq[u].w < ie)) ? 1u : 0u;
                }
            }
            if (r < need) s.sel[base + r] = ie;
        }
        __syncthreads();
        if (tid == 0) s.count = base + need;
        __syncthreads();
        return;
    }
    uint32_t prefix;
    int32_t last;
    later_digits(s, m, d0 >> (kDigitBits - 12), need, [&](int e) { return s.ckey[e]; }, [&](int e) { return s.cidx[e]; },
                 prefix, last);
    uint32_t pos0 = base;
    for (int e0 = 0; e0 < m; e0 += kThreads) {  // uniform trip count (block_scan)
        const int e = e0 + tid;
        bool take = false;
        int32_t c = 0;
        if (e < m) {
            const uint32_t k = s.ckey[e];
            c = s.cidx[e];
            take = k > prefix || (k == prefix && c < last);
        }
        uint32_t tot;
        const uint32_t pos = pos0 + block_scan(take ? 1u : 0u, tot, s.wsum);
        *(take && pos < (uint32_t)kTopkMaxK ? &s.sel[pos] : (int32_t*)&s.trash[0][tid]) = c;
        pos0 += tot;
    }
    __syncthreads();
    if (tid == 0) s.count = pos0;
    __syncthreads();
}

// Writes the K kept indices s.sel[0 .. K) (distinct, all below n) to out in
// ascending order.  For n <= kBitmapMax: a bitmap of the kept indices; each
// thread counts the bits of its stretch of 32 words, a workgroup scan gives
// its first place, and it records the place of each of its words' first bit
// (the running count); then each kept index goes to the place of its word
// plus the number of bits below it in that word.  Otherwise each index goes
// to the place given by the number of kept indices below it.
__device__ __forceinline__ void rank_sort_write(Smem& s, int K, int n, int32_t* out) {
    const int tid = threadIdx.x;
    if (n <= kBitmapMax) {
        const int words = (n + 31) >> 5;
        constexpr int kWpt = kBitmapMax / 32 / kThreads;  // words per thread (32)
        static_assert(kWpt == 32 && kTopkMaxK < 65536, "one bitmap stretch per thread; 16-bit places");
        uint32_t* const bitmap = s.hist;                  // word w at bitmap_word(w)
        uint32_t* const place = s.hist + 36 * kThreads;   // thread t's 32 word places, two 16-bit places per
                                                          // word, at 20 t (16 lanes' 16-byte stores: 16 bank groups)
        const int padded = 36 * ((words + 31) >> 5);
        for (int j = 4 * tid; j < padded; j += 4 * kThreads) *(uint4*)&bitmap[j] = uint4{0u, 0u, 0u, 0u};
        __syncthreads();
        for (int i = tid; i < K; i += kThreads) {
            const int32_t v = s.sel[i];
            atomicOr(&bitmap[bitmap_word(v >> 5)], 1u << (v & 31));
        }
        __syncthreads();
        const int w0 = kWpt * tid;
        uint32_t cnt[kWpt];
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kWpt; j += 4) {
            const uint4 q = w0 + j < words ? *(const uint4*)&bitmap[36 * tid + j] : uint4{0u, 0u, 0u, 0u};
            cnt[j] = w0 + j < words ? __popc(q.x) : 0u;
            cnt[j + 1] = w0 + j + 1 < words ? __popc(q.y) : 0u;
            cnt[j + 2] = w0 + j + 2 < words ? __popc(q.z) : 0u;
            cnt[j + 3] = w0 + j + 3 < words ? __popc(q.w) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kWpt; ++j) mine += cnt[j];
        uint32_t tot;
        uint32_t run = block_scan(mine, tot, s.wsum);
        uint32_t pk[kWpt / 2];
#pragma unroll
        for (int j = 0; j < kWpt; j += 2) {
            const uint32_t lo = run;
            run += cnt[j];
            pk[j / 2] = lo | (run << 16);
            run += cnt[j + 1];
        }
#pragma unroll
        for (int q = 0; q < kWpt / 8; ++q)
            *(uint4*)&place[20 * tid + 4 * q] = uint4{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
        __syncthreads();
        for (int i = tid; i < K; i += kThreads) {
            const int32_t v = s.sel[i];
            const int w = v >> 5;
            const uint32_t word = bitmap[bitmap_word(w)];
            const uint32_t pw = place[20 * (w >> 5) + ((w & 31) >> 1)];
            const uint32_t first = (w & 1) ? pw >> 16 : pw & 0xFFFFu;
            out[first + __popc(word & ((1u << (v & 31)) - 1u))] = v;
        }
        return;
    }
    const int K16 = (K + 15) & ~15;
    for (int j = K + tid; j < K16; j += kThreads) s.sel[j] = INT32_MAX;
    __syncthreads();
    for (int i = tid; i < K; i += kThreads) {
        const int32_t v = s.sel[i];
        uint32_t r = 0;
        for (int j = 0; j < K16; j += 16) {  // 16 bytes per read, 4 reads in flight
            int4 q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = *(const int4*)&s.sel[j + 4 * u];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                r += (q[u].x < v ? 1u : 0u) + (q[u].y < v ? 1u : 0u) + (q[u].z < v ? 1u : 0u) + (q[u].w < v ? 1u : 0u);
        }
        out[r] = v;
    }
}

// One batch of elements: this thread's n_el elements (key, index, valid).
// Counts those above d0 and at d0, places them by one packed workgroup scan,
// and stores: above -> s.sel, at -> s.ckey / s.cidx (at most kCompCap).
template <int n_el, int kDigitBits = 12>
__device__ __forceinline__ void split_batch(Smem& s, uint32_t d0, const uint32_t (&k)[n_el], const int32_t (&c)[n_el],
                                            uint32_t& n_above, uint32_t& n_at) {
    // Elements that do not exist carry key 0, whose digit 0 lies below any
    // threshold digit of existing keys (d0 >= 1).
    constexpr int kSh = 32 - kDigitBits;
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < n_el; ++j) {
        const uint32_t d = k[j] >> kSh;
        cnt += d > d0 ? 1u : (d == d0 ? 0x10000u : 0u);
    }
    uint32_t tot;
    const uint32_t pos = block_scan(cnt, tot, s.wsum);  // both counts < 2^16 per batch
    uint32_t pa = n_above + (pos & 0xFFFFu), pe = n_at + (pos >> 16);
    // Branch-free: every element is stored, to its place or to this lane's
    // trash word (divergent branches per element would cost far more).
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < n_el; ++j) {
        const uint32_t d = k[j] >> kSh;
        const bool a = d > d0 && pa < (uint32_t)kTopkMaxK;
        const bool e = d == d0 && pe < (uint32_t)kCompCap;
        int32_t* ds = a ? &s.sel[pa] : (int32_t*)&s.trash[0][tid];
        uint32_t* dk = e ? &s.ckey[pe] : &s.trash[1][tid];
        int32_t* dc = e ? &s.cidx[pe] : (int32_t*)&s.trash[2][tid];
        *ds = c[j];
        *dk = k[j];
        *dc = c[j];
        pa += d > d0 ? 1u : 0u;
        pe += d == d0 ? 1u : 0u;
    }
    n_above += tot & 0xFFFFu;
    n_at += tot >> 16;
}

// The whole selection among m > K elements (key key_of(e), index idx_of(e)
// below n_all) by one workgroup; writes the K kept indices, ascending, to out.
template <typename KeyOf, typename IdxOf>
__device__ void select_elems(Smem& s, int m, int K, KeyOf key_of, IdxOf idx_of, int n_all, int32_t* out) {
    const int tid = threadIdx.x;
    uint32_t n_eq = 0;
    radix_pass<true, 4096>(s, m, kShift[0], (uint32_t)K, key_of, [](int, uint32_t) { return true; }, &n_eq);
    const uint32_t d0 = s.pick[0];
    const uint32_t need = (uint32_t)K - s.pick[1];
    if (n_eq <= (uint32_t)kCompCap) {
        // The candidates at d0 fit in LDS: one more pass moves them there
        // (and those above d0 to sel).
        uint32_t n_above = 0, n_at = 0;
        for (int c0 = 0; c0 < m; c0 += kThreads * kUnroll) {
            uint32_t k[kUnroll];
            int32_t c[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                const int e = c0 + tid + kThreads * j;
                k[j] = e < m ? key_of(min(e, m - 1)) : 0u;  // key 0: no element (below every digit d0)
                c[j] = idx_of(min(e, m - 1));
            }
            split_batch(s, d0, k, c, n_above, n_at);
        }
        __syncthreads();
        if (tid == 0) s.count = n_above;
        __syncthreads();
        select_at_threshold(s, (int)n_eq, d0, need);
    } else {
        // Heavy ties at d0: the later digits run over all m elements.
        uint32_t prefix;
        int32_t last;
        later_digits(s, m, d0, need, key_of, idx_of, prefix, last);
        uint32_t pos0 = 0;
        for (int c0 = 0; c0 < m; c0 += kThreads * kUnroll) {
            uint32_t k[kUnroll];
            bool take[kUnroll];
            uint32_t cnt = 0;
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) k[j] = key_of(min(c0 + tid + kThreads * j, m - 1));
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                const int e = c0 + tid + kThreads * j;
                const uint32_t d = k[j] >> kShift[0];
                take[j] = e < m && (d > d0 || (d == d0 && (k[j] > prefix || (k[j] == prefix && idx_of(min(e, m - 1)) < last))));
                cnt += take[j] ? 1u : 0u;
            }
            uint32_t tot;
            uint32_t pos = pos0 + block_scan(cnt, tot, s.wsum);
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                if (take[j]) {
                    if (pos < (uint32_t)kTopkMaxK) s.sel[pos] = idx_of(c0 + tid + kThreads * j);
                    ++pos;
                }
            }
            pos0 += tot;
        }
        __syncthreads();
    }
    rank_sort_write(s, K, n_all, out);
}

// The whole selection of one row of n > K candidates by one workgroup.
__device__ void select_row(Smem& s, const float* row, int n, int K, int32_t* out) {
    select_elems(s, n, K, [&](int c) { return score_key(row[c]); }, [](int c) { return c; }, n, out);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    __shared__ Smem s;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int K = a.K;
    const int n = min(a.n_cand[t], a.ld);
    int32_t* out = a.out + (int64_t)t * a.out_ld;
    if (n <= K) {  // every candidate is kept
        for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    select_row(s, a.scores + (int64_t)t * a.s_ld, n, K, out);
}

// ---- multi-workgroup path -------------------------------------------------
constexpr int kChunkThreads = 512;               // threads of a chunk workgroup (8 waves)
constexpr int kPer = kTopkChunk / kChunkThreads;  // candidates per thread of a chunk (32)

// Survivors a chunk stages in LDS (more: the row falls back): K + 1024, in
// the dynamic LDS of the launch, so that small K leaves room for more
// workgroups per compute unit.
__host__ __device__ constexpr int chunk_stage(int K) { return K + 1024; }

// Candidate of lane slot j (of kPer) of thread tid in its chunk: with
// kVec = 4 each thread loads 4 scores at a time (candidates 2048 (j / 4) +
// 4 tid + j % 4), else one (candidate 512 j + tid).
template <int kVec>
__device__ __forceinline__ int chunk_cand(int j, int tid) {
    return kVec == 4 ? 4 * kChunkThreads * (j >> 2) + 4 * tid + (j & 3) : kChunkThreads * j + tid;
}

template <int kVec>
// Four waves per SIMD (at most 128 registers; it takes 99): asking for more
// makes the compiler spill, which measured slower.
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_chunk_kernel(TopkArgs a) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t pick[2];
    __shared__ uint32_t pick_q[2];
    __shared__ uint32_t wsum[kChunkThreads / 64];
    __shared__ uint32_t base;
    __shared__ uint32_t trash[2][64];
    extern __shared__ uint32_t stage[];  // chunk_stage(K) keys, then as many indices
    const int kStage = chunk_stage(a.K);
    uint32_t* const stage_k = stage;
    uint32_t* const stage_c = stage + kStage;
    const int t = blockIdx.y;
    const int n = min(a.n_cand[t], a.ld);
    const int c_lo = blockIdx.x * kTopkChunk;
    if (n <= a.K || c_lo >= n) return;  // the row keeps everything, or the chunk lies past its end
    const int c_hi = min(n, c_lo + kTopkChunk);
    const int tid = threadIdx.x;
    for (int j = tid; j < kBins; j += kChunkThreads) hist[j] = 0;
    // Offsets are taken from the chunk's start (a uniform base), 32-bit and
    // unsigned, so that each load needs one offset register; which of the
    // thread's candidates exist is one 32-bit mask (all of them in a full
    // chunk), so that no per-candidate index stays live across the kernel.
    const float* crow = a.scores + (int64_t)t * a.s_ld + c_lo;
    const uint32_t span = (uint32_t)(c_hi - c_lo);
    constexpr int kMaskWords = (kPer + 31) / 32;
    uint32_t exists[kMaskWords];
#pragma unroll
    for (int q = 0; q < kMaskWords; ++q) exists[q] = ~0u;
    if (span < (uint32_t)kTopkChunk) {
#pragma unroll
        for (int q = 0; q < kMaskWords; ++q) exists[q] = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) exists[j >> 5] |= (uint32_t)((uint32_t)chunk_cand<kVec>(j, tid) < span) << (j & 31);
    }
    auto has = [&](int j) { return (exists[j >> 5] >> (j & 31)) & 1u; };
    uint32_t k[kPer];
    if constexpr (kVec == 4) {
        // 16-byte loads (the launcher checked the alignment); a vector past
        // the chunk's end is clamped to the chunk's last one, which lies
        // within the row's ld scores (ld % 4 == 0).
        const uint32_t last4 = (span - 1) & ~3u;
#pragma unroll
        for (int j = 0; j < kPer; j += 4) {
            const float4 v = *(const float4*)(crow + min((uint32_t)chunk_cand<4>(j, tid), last4));
            k[j] = score_key(v.x);
            k[j + 1] = score_key(v.y);
            k[j + 2] = score_key(v.z);
            k[j + 3] = score_key(v.w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) k[j] = score_key(crow[min((uint32_t)chunk_cand<1>(j, tid), span - 1)]);
    }
    __syncthreads();
    // Plain atomics: at most 64 per lane, so even a chunk of equal keys
    // serialises for a bounded time.
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (has(j)) atomicAdd(&hist[k[j] >> kShift[0]], 1u);
    __syncthreads();
    pick_digit<true, kBins, kChunkThreads>(hist, (uint32_t)min(a.K, c_hi - c_lo), pick, wsum);
    // A full chunk's share of the row's threshold bound: its q-th best digit.
    const int full_chunks = n / kTopkChunk;
    const bool full = c_hi - c_lo == kTopkChunk;
    if (full) pick_digit<true, kBins, kChunkThreads>(hist, (uint32_t)((a.K + full_chunks - 1) / full_chunks), pick_q, wsum);
    __syncthreads();
    const uint32_t d0 = pick[0];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += (has(j) && (k[j] >> kShift[0]) >= d0) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = block_scan<kChunkThreads>(mine, tot, wsum);
    uint32_t base0 = 0;
    if (tid == 0) {
        base0 = atomicAdd(&a.ws_count[4 * t], tot);
        if (tot > (uint32_t)kStage) atomicOr(&a.ws_count[4 * t + 1], 1u);  // the row's list is incomplete
        if (full) atomicMax(&a.ws_count[4 * t + 2], (uint32_t)kBins - pick_q[0]);  // kBins - min_c d_c
    }
    // The survivors into LDS (branch-free: the others go to this lane's trash
    // word), then to the row's list with coalesced stores.  The list offset
    // is waited for only after the LDS stores (this file is built without the
    // compiler's atomic combining, which would wait for it right away).  (The thread index
    // is re-read, so that the candidate indices are recomputed here rather
    // than kept from the loads.)
    int tid_again = tid;
    asm volatile("" : "+v"(tid_again));
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int c = c_lo + chunk_cand<kVec>(j, tid_again);
        const bool take = has(j) && (k[j] >> kShift[0]) >= d0;
        const bool keep = take && pos < (uint32_t)kStage;
        *(keep ? &stage_k[pos] : &trash[0][tid & 63]) = k[j];
        *(keep ? &stage_c[pos] : &trash[1][tid & 63]) = (uint32_t)c;
        pos += take ? 1u : 0u;
    }
    if (tid == 0) base = base0;
    __syncthreads();
    const int64_t cap = a.ws_cap;
    uint64_t* list = a.ws_list + (int64_t)t * cap;
    const int64_t b = base;
    const int n_st = (int)min(tot, (uint32_t)kStage);  // a larger total overflows the row's list anyway
    for (int i = tid; i < n_st; i += kChunkThreads)
        if (b + i < cap) list[b + i] = ((uint64_t)stage_k[i] << 32) | stage_c[i];
}

constexpr int kLB = 24;  // 16-byte list loads (two entries each) per thread per batch

// This thread's entries of list batch b0 (pairs b0 + tid + 256*j): key and
// index, key 0 for an entry past the list's end (no finite score has key 0:
// the lowest is 0x00800000, so such an entry never reaches a threshold
// digit).  The list's rows are 16-byte aligned (even capacity); an entry is
// (key << 32) | index.
__device__ __forceinline__ void load_list_pairs(const uint64_t* list, int n2, int b0, uint4 (&q)[kLB]) {
    const uint4* l4 = (const uint4*)list;
#pragma unroll
    for (int j = 0; j < kLB; ++j) q[j] = l4[min(b0 + (int)threadIdx.x + kThreads * j, n2 - 1)];
}

__device__ __forceinline__ void unpack_list_pairs(const uint4 (&q)[kLB], int m, int b0, uint32_t (&k)[2 * kLB],
                                                  int32_t (&c)[2 * kLB]) {
#pragma unroll
    for (int j = 0; j < kLB; ++j) {
        const int e = 2 * (b0 + (int)threadIdx.x + kThreads * j);
        k[2 * j] = e < m ? q[j].y : 0u;
        c[2 * j] = (int32_t)q[j].x;
        k[2 * j + 1] = e + 1 < m ? q[j].w : 0u;
        c[2 * j + 1] = (int32_t)q[j].z;
    }
}

__device__ __forceinline__ void load_list_batch(const uint64_t* list, int m, int b0, uint32_t (&k)[2 * kLB],
                                                int32_t (&c)[2 * kLB]) {
    uint4 q[kLB];
    load_list_pairs(list, (m + 1) >> 1, b0, q);
    unpack_list_pairs(q, m, b0, k, c);
}

__global__ __launch_bounds__(kThreads) void topk_finish_kernel(TopkArgs a) {
    __shared__ Smem s;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int K = a.K;
    const int n = min(a.n_cand[t], a.ld);
    int32_t* out = a.out + (int64_t)t * a.out_ld;
    if (n <= K) {  // every candidate is kept
        for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    // The list's first batch goes out with the counters (bounded by the
    // capacity, masked by the count once it is known).
    const uint64_t* list = a.ws_list + (int64_t)t * a.ws_cap;
    uint4 q0[kLB];
    load_list_pairs(list, (int)(a.ws_cap >> 1), 0, q0);
    const uint32_t m = a.ws_count[4 * t];
    const bool overflow = a.ws_count[4 * t + 1] != 0u;
    const uint32_t bound = a.ws_count[4 * t + 2];
    __syncthreads();  // every thread has read the counters
    if (tid == 0) {   // zero for the next call
        a.ws_count[4 * t] = 0u;
        a.ws_count[4 * t + 1] = 0u;
        a.ws_count[4 * t + 2] = 0u;
    }
    if (overflow || (int64_t)m > a.ws_cap) {  // the list is incomplete: the whole row
        select_row(s, a.scores + (int64_t)t * a.s_ld, n, K, out);
        return;
    }
    const int m2 = ((int)m + 1) >> 1;
    if (bound != 0u && m2 <= kThreads * kLB) {
        // The entries at or above the bound digit lb (kept in registers and
        // then in LDS, in the fine histogram's upper bins) hold the row's top
        // K.  Their keys span [lb << 20, kmax]; one histogram over that span
        // cut into at most kBins bins (the key offset from lb << 20, shifted
        // right by sh) usually leaves a handful of candidates in the
        // threshold bin, which are then ranked directly.
        const uint32_t lb = (uint32_t)kBins - bound;
        uint32_t* ck = s.hist + kBins;
        int32_t* ci = (int32_t*)(s.hist + 2 * kBins);
        uint32_t k[2 * kLB];
        int32_t c[2 * kLB];
        unpack_list_pairs(q0, (int)m, 0, k, c);
        uint32_t cnt = 0, kmax = 0;
#pragma unroll
        for (int j = 0; j < 2 * kLB; ++j) {
            const bool in = k[j] != 0u && (k[j] >> kShift[0]) >= lb;  // key 0: no entry
            cnt += in ? 1u : 0u;
            kmax = in ? max(kmax, k[j]) : kmax;
        }
        if (tid == 0) s.kmax = 0u;
        uint32_t tot;
        uint32_t pos = block_scan(cnt, tot, s.wsum);  // (its barriers order the store above)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
        if ((tid & 63) == 0) atomicMax(&s.kmax, kmax);
        if (tot <= (uint32_t)kCompCap) {
#pragma unroll
            for (int j = 0; j < 2 * kLB; ++j) {
                if (k[j] != 0u && (k[j] >> kShift[0]) >= lb) {
                    ck[pos] = k[j];
                    ci[pos] = c[j];
                    ++pos;
                }
            }
        }
        __syncthreads();
        if (tot > (uint32_t)K && tot <= (uint32_t)kCompCap) {  // tot >= K always; tot == K: the general route
            const uint32_t base = lb << kShift[0];
            const uint32_t span = s.kmax - base;
            const int sh = max(0, 20 - __clz((int)span));  // (span >> sh) < kBins
            for (int j = tid; j < kBins; j += kThreads) s.hist[j] = 0u;
            __syncthreads();
            for (int e = tid; e < (int)tot; e += kThreads) atomicAdd(&s.hist[(ck[e] - base) >> sh], 1u);
            __syncthreads();
            pick_digit<true, kBins>(s.hist, (uint32_t)K, s.pick, s.wsum);
            __syncthreads();
            const uint32_t dt = s.pick[0];
            const uint32_t need = (uint32_t)K - s.pick[1];
            const uint32_t n_eq = s.hist[dt];
            if (n_eq <= (uint32_t)kRankMax) {
                // Above the threshold bin: kept; in it: ranked.
                constexpr int kPerT = kCompCap / kThreads;
                uint32_t bk[kPerT], bcnt = 0;
                int32_t bc[kPerT];
#pragma unroll
                for (int j = 0; j < kPerT; ++j) {
                    const int e = tid + kThreads * j;
                    bk[j] = e < (int)tot ? ck[e] : base;  // no entry: bin 0 -> neither (dt > 0 or n_eq counts it)
                    bc[j] = ci[min(e, (int)tot - 1)];
                    const uint32_t d = (bk[j] - base) >> sh;
                    bcnt += e < (int)tot ? (d > dt ? 1u : (d == dt ? 0x10000u : 0u)) : 0u;
                }
                uint32_t btot;
                const uint32_t bpos = block_scan(bcnt, btot, s.wsum);
                uint32_t pa = bpos & 0xFFFFu, pe = bpos >> 16;
#pragma unroll
                for (int j = 0; j < kPerT; ++j) {
                    const int e = tid + kThreads * j;
                    const uint32_t d = (bk[j] - base) >> sh;
                    if (e < (int)tot && d > dt) s.sel[pa++] = bc[j];
                    if (e < (int)tot && d == dt) {
                        s.ckey[pe] = bk[j];
                        s.cidx[pe] = bc[j];
                        ++pe;
                    }
                }
                __syncthreads();
                if (tid == 0) s.count = btot & 0xFFFFu;
                __syncthreads();
                select_at_threshold(s, (int)n_eq, 0u, need);  // n_eq <= kRankMax: by rank
                rank_sort_write(s, K, n, out);
                return;
            }
            __syncthreads();  // hist is cleared below
        }
    }
    for (int j = 4 * tid; j < kFineBins; j += 4 * kThreads) *(uint4*)&s.hist[j] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    uint32_t n_above = 0, n_at = 0, d0 = 0, need = 0, n_eq = 0;
    bool whole_row = false;
    if (m2 <= kThreads * kLB) {
        // The whole list in one batch of loads, kept in registers for both
        // the first digit's histogram and the split.
        uint32_t k[2 * kLB];
        int32_t c[2 * kLB];
        unpack_list_pairs(q0, (int)m, 0, k, c);
#pragma unroll
        for (int j = 0; j < 2 * kLB; ++j) atomicAdd(&s.hist[k[j] >> (32 - kFineBits)], 1u);  // key 0: bin 0, below all
        __syncthreads();
        pick_digit<true, kFineBins>(s.hist, (uint32_t)K, s.pick, s.wsum);
        __syncthreads();
        d0 = s.pick[0];
        need = (uint32_t)K - s.pick[1];
        n_eq = s.hist[d0];
        whole_row = n_eq > (uint32_t)kCompCap;
        if (!whole_row) split_batch<2 * kLB, kFineBits>(s, d0, k, c, n_above, n_at);
    } else {
        for (int b0 = 0; b0 < m2; b0 += kThreads * kLB) {
            uint32_t k[2 * kLB];
            int32_t c[2 * kLB];
            load_list_batch(list, (int)m, b0, k, c);
#pragma unroll
            for (int j = 0; j < 2 * kLB; ++j) atomicAdd(&s.hist[k[j] >> (32 - kFineBits)], 1u);
        }
        __syncthreads();
        pick_digit<true, kFineBins>(s.hist, (uint32_t)K, s.pick, s.wsum);
        __syncthreads();
        d0 = s.pick[0];
        need = (uint32_t)K - s.pick[1];
        n_eq = s.hist[d0];
        whole_row = n_eq > (uint32_t)kCompCap;
        if (!whole_row) {
            for (int b0 = 0; b0 < m2; b0 += kThreads * kLB) {
                uint32_t k[2 * kLB];
                int32_t c[2 * kLB];
                load_list_batch(list, (int)m, b0, k, c);
                split_batch<2 * kLB, kFineBits>(s, d0, k, c, n_above, n_at);
            }
        }
    }
    if (whole_row) {  // heavy ties at the threshold digit: the whole row
        select_row(s, a.scores + (int64_t)t * a.s_ld, n, K, out);
        return;
    }
    __syncthreads();
    if (tid == 0) s.count = n_above;
    __syncthreads();
    select_at_threshold<kFineBits>(s, (int)n_eq, d0, need);
    rank_sort_write(s, K, n, out);
}

}  // namespace

int64_t topk_list_cap(int64_t ld, int64_t K) {
    const int64_t chunks = (ld + kTopkChunk - 1) / kTopkChunk;
    const int64_t cap = chunks * std::min<int64_t>(kTopkChunk, chunk_stage((int)K));
    return (cap + 1) & ~(int64_t)1;  // even: rows stay 16-byte aligned
}

size_t topk_workspace_bytes(int64_t T, int64_t ld, int64_t K) {
    if (ld < kTopkSplitMin) return 0;
    return (size_t)T * (size_t)topk_list_cap(ld, K) * 8;
}

void topk_bind_workspace(TopkArgs& a, void* ws, uint32_t* counters) {
    a.ws_cap = topk_list_cap(a.ld, a.K);
    a.ws_list = (uint64_t*)ws;
    a.ws_count = counters;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    if (a.ws_list == nullptr) {
        hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.T), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.ld + kTopkChunk - 1) / kTopkChunk), (unsigned)a.T);
    const size_t stage_bytes = 2 * sizeof(uint32_t) * (size_t)chunk_stage(a.K);
    // 16-byte loads need aligned rows, and a row width that is a multiple of
    // 4 (a vector never reaches past a row's last score).
    if (((uintptr_t)a.scores & 15) == 0 && (a.s_ld & 3) == 0 && (a.ld & 3) == 0)
        hipLaunchKernelGGL(topk_chunk_kernel<4>, grid, dim3(kChunkThreads), stage_bytes, stream, a);
    else
        hipLaunchKernelGGL(topk_chunk_kernel<1>, grid, dim3(kChunkThreads), stage_bytes, stream, a);
    hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.T), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsv4
