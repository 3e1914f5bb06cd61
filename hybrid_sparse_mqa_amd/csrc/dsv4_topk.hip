// dsv4_topk.hip -- C4 top-k selection: for every query row, the K candidate
// compressed entries with the highest indexer scores (the DeepSeek-V4 /
// SGLang overview page: the indexer keeps the top 512 compressed entries per
// query, its kernel section naming a Lightning TopK kernel), produced as the
// c4_indices the attention reads.  Equal scores: the lower index wins, and
// -0.0 equals +0.0.  Output: the kept indices in ascending order, then -1.
//
// One workgroup per row, a radix select on 32-bit keys that order like the
// scores: three passes of 12-, 10- and 10-bit histograms in LDS over the
// candidates that still match the key prefix fix the threshold key and how
// many of the candidates equal to it are kept; when fewer than all of those
// are kept, a second radix select on their indices finds the last one kept.
// The kept indices are then appended to an LDS list and sorted (bitonic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_launch.h"

namespace dsv4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// Order-preserving key: a > b as scores (with -0 == +0) iff key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x + 0.0f);  // -0.0 + 0.0 = +0.0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kBins = 4096;     // digits of 12, 10 and 10 bits
constexpr int kCompCap = 4096;  // candidates kept in LDS after the first pass

// Adds one to hist[bin] for the active lanes.  The lanes that share the first
// active lane's bin add with one atomic: keys concentrated in a few bins (a
// narrow score range, ties) would otherwise serialise on one LDS address.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int first = __builtin_ctzll(act);
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
    const uint64_t same = __ballot(active && bin == b0);
    if (active && bin != b0) atomicAdd(&hist[bin], 1u);
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], (uint32_t)__popcll(same));
}

// Wave 0 picks the digit of one radix pass from hist[0 .. nb).  Descending
// (top keys): the largest d with count(digit >= d) >= need; out[1] =
// count(digit > d).  Ascending (low indices): the smallest d with
// count(digit <= d) >= need; out[1] = count(digit < d).  out[0] = d.
// need >= 1 and the histogram total >= need.
template <bool kDescending>
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nb, uint32_t need, uint32_t* out) {
    const int l = threadIdx.x & 63;
    const int per = nb / 64;
    const uint32_t* my = hist + per * l;
    uint32_t mine = 0;
    for (int j = 0; j < per; ++j) mine += my[j];
    uint32_t incl = mine;  // sum over lanes <= l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t up = __shfl_up(incl, o);
        if (l >= o) incl += up;
    }
    const uint32_t total = __shfl(incl, 63);
    uint32_t le = incl - mine;  // count(digit < per*l)
    int pick = -1;
    uint32_t skip = 0;
    for (int j = 0; j < per; ++j) {
        const uint32_t bin = my[j];
        le += bin;  // count(digit <= per*l + j)
        if (kDescending) {
            if (total - le + bin >= need) {  // count(digit >= d): the largest such d
                pick = j;
                skip = total - le;
            }
        } else if (pick < 0 && le >= need) {  // the smallest such d
            pick = j;
            skip = le - bin;
        }
    }
    const uint64_t ok = __ballot(pick >= 0);
    const int lane = kDescending ? 63 - __builtin_clzll(ok) : __builtin_ctzll(ok);
    if (l == lane) {
        out[0] = (uint32_t)(per * l + pick);
        out[1] = skip;
    }
}

// One radix pass: the histogram of digit (v >> shift) & (nb-1) over the
// candidates c < n for which `match` holds (v = key_of(c)), then the pick.
// Leaves the digit in pick[0], the skipped count in pick[1] and the chosen
// bin's count in *n_bin (for every thread).
template <bool kDescending, typename KeyOf, typename Match>
__device__ __forceinline__ void radix_pass(uint32_t* hist, uint32_t* pick, int n, int shift, int nb, uint32_t need,
                                           KeyOf key_of, Match match, uint32_t* n_bin) {
    const int tid = threadIdx.x;
    for (int j = tid; j < nb; j += kThreads) hist[j] = 0;
    __syncthreads();
    // kUnroll candidates per thread per step, all loaded before any is used
    // (one load round trip per step, not per candidate); a uniform trip
    // count, so every lane reaches the ballots.
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
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) hist_add(hist, (v[j] >> shift) & (uint32_t)(nb - 1), m[j]);
    }
    __syncthreads();
    if (tid < 64) pick_digit<kDescending>(hist, nb, need, pick);
    __syncthreads();
    *n_bin = hist[pick[0]];
    __syncthreads();  // hist and pick are reused by the next pass
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t pick[2];
    __shared__ uint32_t count;
    __shared__ int32_t sel[kTopkMaxK];
    __shared__ uint32_t ckey[kCompCap];
    __shared__ int32_t cidx[kCompCap];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int K = a.K;
    const int n = min(a.n_cand[t], a.ld);
    const float* row = a.scores + (int64_t)t * a.s_ld;
    int32_t* out = a.out + (int64_t)t * a.out_ld;
    if (n <= K) {  // every candidate is kept
        for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }

    // Threshold key: prefix of the keys fixed so far, and how many of the
    // candidates matching it are still to be kept.  Digits of 12, 10, 10 bits.
    constexpr int kShift[3] = {20, 10, 0}, kNb[3] = {4096, 1024, 1024};
    uint32_t prefix = 0, pmask = 0, need = (uint32_t)K, n_eq = 0;
    auto key_of = [&](int c) { return score_key(row[c]); };
    radix_pass<true>(hist, pick, n, kShift[0], kNb[0], need, key_of, [](int, uint32_t) { return true; }, &n_eq);
    const uint32_t d0 = pick[0];
    need -= pick[1];
    // The candidates whose first digit is d0 or above: every one that can be
    // kept.  Usually few; then they move to LDS (key, index) and the other
    // passes and the selection run there instead of over all n candidates.
    const uint32_t n_top = pick[1] + n_eq;
    const bool compact = n_top <= (uint32_t)kCompCap;
    prefix = d0 << kShift[0];
    pmask = (uint32_t)(kNb[0] - 1) << kShift[0];
    if (compact) {
        if (tid == 0) count = 0;
        __syncthreads();
        for (int c0 = 0; c0 < n; c0 += kThreads * kUnroll) {
            uint32_t k[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) k[j] = key_of(min(c0 + tid + kThreads * j, n - 1));
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                const int c = c0 + tid + kThreads * j;
                if (c < n && (k[j] >> kShift[0]) >= d0) {
                    const uint32_t pos = atomicAdd(&count, 1u);  // exactly n_top of them (bounded for safety)
                    if (pos < (uint32_t)kCompCap) {
                        ckey[pos] = k[j];
                        cidx[pos] = c;
                    }
                }
            }
        }
        __syncthreads();
    }
    const int m = compact ? (int)n_top : n;  // elements the remaining passes walk
    auto elem_key = [&](int e) { return compact ? ckey[e] : key_of(e); };
    auto elem_idx = [&](int e) { return compact ? cidx[e] : e; };
    for (int p = 1; p < 3; ++p) {
        const uint32_t pm = pmask, pf = prefix;
        radix_pass<true>(hist, pick, m, kShift[p], kNb[p], need, elem_key,
                         [=](int, uint32_t v) { return (v & pm) == pf; }, &n_eq);
        need -= pick[1];
        prefix |= pick[0] << kShift[p];
        pmask |= (uint32_t)(kNb[p] - 1) << kShift[p];
    }
    // Keep every key above `prefix` and the first `need` (by index) equal to it.
    int32_t last = n;  // keep equal keys with index < last
    if (need < n_eq) {
        uint32_t ip = 0, imask = 0, ineed = need, n_in = 0;
        const uint32_t T = prefix;
        for (int p = 0; p < 3; ++p) {
            const uint32_t im = imask, ipf = ip;
            radix_pass<false>(hist, pick, m, kShift[p], kNb[p], ineed, [&](int e) { return (uint32_t)elem_idx(e); },
                              [&, T, im, ipf](int e, uint32_t v) { return elem_key(e) == T && (v & im) == ipf; }, &n_in);
            ineed -= pick[1];
            ip |= pick[0] << kShift[p];
            imask |= (uint32_t)(kNb[p] - 1) << kShift[p];
        }
        last = (int32_t)ip + 1;  // the need-th equal key is at index ip
    }
    if (tid == 0) count = 0;
    __syncthreads();
    for (int e0 = 0; e0 < m; e0 += kThreads * kUnroll) {
        uint32_t k[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) k[j] = elem_key(min(e0 + tid + kThreads * j, m - 1));
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int e = e0 + tid + kThreads * j;
            if (e < m) {
                const int32_t c = elem_idx(e);
                if (k[j] > prefix || (k[j] == prefix && c < last)) {
                    const uint32_t pos = atomicAdd(&count, 1u);  // exactly K of them (bounded for safety)
                    if (pos < (uint32_t)kTopkMaxK) sel[pos] = c;
                }
            }
        }
    }
    __syncthreads();  // count == K
    int P = 1;
    while (P < K) P <<= 1;
    for (int j = K + tid; j < P; j += kThreads) sel[j] = INT32_MAX;
    __syncthreads();
    // Bitonic sort of sel[0 .. P) ascending.
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += kThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const int32_t x = sel[lo], y = sel[hi];
                if ((x > y) == up) {
                    sel[lo] = y;
                    sel[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int j = tid; j < K; j += kThreads) out[j] = sel[j];
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.T), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsv4
