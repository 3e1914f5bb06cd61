// dsv4_launch.h -- argument blocks and launch entry points of the HIP kernels
// (internal to the library; the public ABI is include/dsv4_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_device.h"

namespace dsv4 {

constexpr int kTileKeys = 32;        // keys per LDS tile
constexpr int kMaxSplitKeys = 1024;  // keys one workgroup may own (LDS slot list)
constexpr int kWideHeadsPerBlock = 64;  // query heads per workgroup, 64-head bf16 and FP8 layouts
constexpr int kWide32HeadsPerBlock = 32;  // query heads per workgroup, 32-head bf16 (both) and FP8 layouts
constexpr int kNarrowHeadsPerBlock = 16;  // query heads per workgroup, narrow bf16 kernel
constexpr int kNarrowTileKeys = 16;       // keys per LDS tile of the narrow kernel
constexpr int kNarrowMaxSplitKeys = 2048; // keys one narrow workgroup may own

// Which split kernel runs: bf16 with 64 heads per workgroup (waves split
// into two head groups x two dim halves), bf16 with 32 heads per workgroup
// (four dim quarters, or score and PV roles), bf16 with 16 heads per
// workgroup (four independent waves), or packed FP8 with 64 heads (two head
// groups x two dim halves) or 32 heads (four dim quarters) per workgroup.
enum class Layout { kWide, kWide32, kRoles32, kNarrow, kFp8, kFp8H32 };
constexpr int kTableCap = 1024;      // extra page-table entries a workgroup caches in LDS
constexpr int kStages = 4;           // bf16 key tiles resident in LDS

struct AttnArgs {
    Meta m;
    const uint16_t* q;  // bf16 [T, H, 512]
    int64_t q_s0, q_s1;
    const uint8_t* swa_pool;  // bf16 rows or packed FP8 pages
    int64_t swa_row_bytes;    // bf16: bytes between rows (>= 1024)
    const uint8_t* ext_pool;
    int64_t ext_row_bytes;
    const float* sink;        // [H] or null
    int32_t T, H;
    float scale_log2;         // scale * log2(e)
    int32_t chunk;            // keys per split (multiple of kTileKeys)
    int32_t splits;           // splits per (row, head block)
    int32_t head_blocks;      // ceil(H / heads per block of the kernel)
    int32_t n_items;          // T * head_blocks * splits work items
    int32_t ext_pages;        // extra page-table width (0 when R == 0)
    uint16_t* out;            // bf16 [T, H, 512]
    int64_t out_s0, out_s1;
    float* lse;               // [T, H] or null
    int64_t lse_s0;
    uint16_t* ws_o;           // bf16 [T, splits, H, 512] normalised partial outputs
    float* ws_lse;            // [T, splits, H] base-2 partial log-sum-exp
    const uint8_t* zero_row;  // >= 1 KiB of zeros, read in place of unused keys
    // Test hook (null in normal calls; then the plain kernel builds run): the
    // recording builds write, for work item (t, hb, s) and split key k, the
    // address of the KV row they copied into dbg_keys[((t * head_blocks + hb)
    // * splits + s) * chunk + k], and the masking kernels the valid-key mask
    // of each 32-key tile into dbg_masks[(...) * 32 + tile].
    uint64_t* dbg_keys;
    uint32_t* dbg_masks;
};

struct GatherArgs {
    Meta m;
    int32_t T;
    int32_t* slots;  // [T, slots_ld]
    int64_t slots_ld;
    int32_t* counts;  // [T, 2]
};

// KV store: n K rows (bf16 [n, 512], row stride k_s0) into packed FP8
// records of the pool at slots[i] (skipped if < 0).
struct PackArgs {
    const uint16_t* k;
    int64_t k_s0;
    const int32_t* slots;  // [n]
    int64_t n;
    uint8_t* pool;         // [pages, page_bytes]
    int64_t page_bytes;
};

// C4 top-k: per row t, the K highest of scores[t][0 .. n_cand[t]) (ties: the
// lower index), ascending, then -1, into out[t][0 .. K).
constexpr int kTopkMaxK = 2048;
constexpr int kTopkBins = 4096;      // first radix digit: the top 12 key bits
constexpr int kTopkChunk = 16384;    // candidates per workgroup, multi-workgroup path
constexpr int kTopkSplitMin = 32768; // rows this long (ld) take the multi-workgroup path
struct TopkArgs {
    const float* scores;  // [T, s_ld]
    int64_t s_ld;
    const int32_t* n_cand;  // [T]
    int32_t* out;           // [T, out_ld]
    int64_t out_ld;
    int32_t T, K, ld;       // ld: candidates per row available (n_cand is clamped to it)
    // Multi-workgroup path (ws_list null: one workgroup per row).  The
    // counters are zero between calls (zeroed when the workspace is
    // allocated, and by the finishing kernel after use).
    uint64_t* ws_list;   // [T, ws_cap] (key << 32) | index of each chunk's survivors
    int64_t ws_cap;
    uint32_t* ws_count;  // [T, 4]: survivors appended so far, list-incomplete flag, threshold bound (kBins - digit, 0: none), unused
};
// List workspace bytes of the multi-workgroup path for T rows (0 if ld is
// short); binding takes the list workspace and the per-row counters.
size_t topk_workspace_bytes(int64_t T, int64_t ld, int64_t K);
void topk_bind_workspace(TopkArgs& a, void* ws, uint32_t* counters);

hipError_t launch_attention(const AttnArgs& a, Layout layout, hipStream_t stream);
hipError_t launch_merge(const AttnArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& g, hipStream_t stream);
hipError_t launch_pack_fp8(const PackArgs& p, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

}  // namespace dsv4
