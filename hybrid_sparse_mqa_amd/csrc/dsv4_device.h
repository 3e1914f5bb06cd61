// dsv4_device.h -- device-side types and the row / key-list indexing shared by
// the gather stage and the fused attention kernel (gfx950).
//
// Row resolution and key lists follow the DeepSeek-V4 attention walk-through
// (sections 1, 4 and 5) and the DSV4 test-matrix page (page size 256):
//   row t -> request r (qo_indptr[r] <= t < qo_indptr[r+1]),
//   position p = seq_lens[r] - n_q + (t - qo_indptr[r]);
//   key list = window positions p-n_swa+1 .. p (n_swa = min(W, p+1)), then
//   the extra list: C4 -> c4_indices[t][0..K) (entries < 0 unused),
//   C128 -> entries 0 .. (p+1)/128 - 1;
//   logical position x -> slot table[r][x >> 8] * 256 + (x & 255).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

constexpr int kHeadDim = 512;
constexpr int kNope = 448;
constexpr int kRope = 64;
constexpr int kPage = 256;
constexpr int kFp8RecBytes = 576;
constexpr int kFp8ScaleOffset = kPage * kFp8RecBytes;  // 147456
constexpr int kFp8PageBytes = kPage * 584;              // 149504

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Metadata of one call, shared by every kernel that walks key lists.
struct Meta {
    const int32_t* seq_lens;   // [B]
    const int32_t* qo_indptr;  // [B+1]
    const int32_t* swa_table;  // [B, swa_ld]
    int64_t swa_ld;
    const int32_t* ext_table;  // [B, ext_ld] (R != 0)
    int64_t ext_ld;
    const int32_t* c4;         // [T, c4_ld] (R == 4)
    int64_t c4_ld;
    int32_t K;                 // C4 list width
    int32_t B, R, W;
};

struct RowKeys {
    int r;       // request
    int p;       // position of the row
    int n_swa;   // window keys
    int swa_lo;  // first window position
    int n_ext;   // extra list length (C4: K entries including unused ones)
};

// Bounds and length of 64 consecutive requests, one per lane.
struct RequestChunk {
    int lo, hi, len;
};

// Lanes past B load request B-1 (every load is unconditional, so no branch
// splits them and a later wait counts them exactly); callers mask those
// lanes out.
__device__ __forceinline__ RequestChunk load_requests(const Meta& m, int base, int lane) {
    const int i = min(base + lane, m.B - 1);
    RequestChunk c;
    c.lo = m.qo_indptr[i];
    c.hi = m.qo_indptr[i + 1];
    c.len = m.seq_lens[i];
    return c;
}

// Row resolution by one wave.  Lane i of each 64-request chunk loads
// qo_indptr[i], qo_indptr[i+1] and seq_lens[i] together; the owning request
// is the last i with qo_indptr[i] <= t (a ballot), and its values are read
// from that lane, so the whole lookup costs one round of loads per chunk.
// `first` is the chunk of requests 0..63, loaded by the caller (which may
// issue other loads before using it); `lane` is the caller's lane id; the
// result is clamped to the batch.
__device__ __forceinline__ RowKeys row_keys_from(const Meta& m, int t, int lane, RequestChunk c) {
    int r = 0, q_lo = 0, q_hi = 0, len = 0;
    auto scan = [&](int base, const RequestChunk& cc) {
        const bool in = base + lane < m.B;
        const uint64_t le = __ballot(in && cc.lo <= t);
        if (le != 0ull) {
            const int src = 63 - __clzll(le);
            r = base + src;
            q_lo = __shfl(cc.lo, src);
            q_hi = __shfl(cc.hi, src);
            len = __shfl(cc.len, src);
        }
    };
    // The first chunk outside any loop, so that waiting for it does not
    // wait for loads the caller issued after it.
    scan(0, c);
    for (int base = 64; base < m.B; base += 64) scan(base, load_requests(m, base, lane));
    RowKeys k;
    k.r = r;
    const int n_q = q_hi - q_lo;
    k.p = len - n_q + (t - q_lo);
    k.n_swa = min(m.W, k.p + 1);
    k.swa_lo = k.p + 1 - k.n_swa;
    k.n_ext = m.R == 4 ? m.K : (m.R == 128 ? (k.p + 1) / 128 : 0);
    return k;
}

__device__ __forceinline__ RowKeys row_keys(const Meta& m, int t, int lane) {
    return row_keys_from(m, t, lane, load_requests(m, 0, lane));
}

// Physical slot of entry i of row t's key list; -1 for an unused C4 entry.
// Entries i < n_swa live in the SWA pool, the others in the extra pool.
__device__ __forceinline__ int32_t list_slot(const Meta& m, const RowKeys& k, int t, int i) {
    if (i < k.n_swa) {
        const int x = k.swa_lo + i;
        return m.swa_table[(int64_t)k.r * m.swa_ld + (x >> 8)] * kPage + (x & (kPage - 1));
    }
    const int e = i - k.n_swa;
    const int c = (m.R == 4) ? m.c4[(int64_t)t * m.c4_ld + e] : e;
    if (c < 0) return -1;
    return m.ext_table[(int64_t)k.r * m.ext_ld + (c >> 8)] * kPage + (c & (kPage - 1));
}

}  // namespace dsv4
