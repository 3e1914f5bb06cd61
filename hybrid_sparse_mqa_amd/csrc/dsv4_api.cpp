// dsv4_api.cpp -- host side of the C ABI declared in include/dsv4_attn.h:
// argument validation (no device reads), split planning from static bounds,
// the per-device workspace for split partials, kernel launches on the caller's
// stream, optional HIP-event timing and the DSV4_VALIDATE contract check.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsv4_attn.h"
#include "dsv4_launch.h"
#include "dsv4_probe.h"

using namespace dsv4;

// 4 KiB of zeros in each device's copy of the code object (zero-initialised
// at load): unused C4 entries and keys past a split read it, so every copy
// stays in bounds and masked keys contribute zeros.  No kernel writes it.
// (Not const: the device compiler drops const device data that no device code
// references, and the runtime then has no device symbol for the host's.)
static __device__ __attribute__((aligned(256))) uint8_t g_zero_row[4096];

// Split partials of dsv4_attn_forward_noalloc, for callers that cannot
// allocate: one copy per device, held until the process ends.  Host code
// must never pass `scratch` itself to a kernel (that is a host-side stand-in):
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

dsv4_status fail(dsv4_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

#define DSV4_TRY(expr)                         \
    do {                                       \
        dsv4_status st_ = (expr);              \
        if (st_ != DSV4_OK) return st_;        \
    } while (0)

#define DSV4_HIP(expr)                                                                       \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess) return fail(DSV4_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

const char* dtype_name(int32_t d) {
    switch (d) {
        case DSV4_BF16: return "bf16";
        case DSV4_F32: return "f32";
        case DSV4_I32: return "i32";
        case DSV4_U8: return "u8";
        default: return "?";
    }
}

// Shape / dtype / stride checks of one descriptor.  shape entries < 0 mean
// "any"; the last dimension must be contiguous.
dsv4_status check_tensor(const char* name, const dsv4_tensor* t, int32_t dtype, int32_t ndim,
                         std::initializer_list<int64_t> shape) {
    if (t == nullptr) return fail(DSV4_ERR_INVALID, "%s: NULL descriptor", name);
    if (t->data == nullptr) return fail(DSV4_ERR_INVALID, "%s: NULL data pointer", name);
    if (t->dtype != dtype)
        return fail(DSV4_ERR_INVALID, "%s: dtype %s, expected %s", name, dtype_name(t->dtype), dtype_name(dtype));
    if (t->ndim != ndim) return fail(DSV4_ERR_INVALID, "%s: ndim %d, expected %d", name, t->ndim, ndim);
    int i = 0;
    int64_t numel = 1;
    for (int d = 0; d < ndim; ++d) numel *= t->shape[d] > 0 ? t->shape[d] : 0;
    for (int64_t s : shape) {
        if (t->shape[i] < 0) return fail(DSV4_ERR_INVALID, "%s: negative extent in dim %d", name, i);
        if (s >= 0 && t->shape[i] != s)
            return fail(DSV4_ERR_INVALID, "%s: dim %d is %lld, expected %lld", name, i, (long long)t->shape[i],
                        (long long)s);
        ++i;
    }
    if (numel == 0) return DSV4_OK;  // empty tensors carry arbitrary strides and are never read
    if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1)
        return fail(DSV4_ERR_INVALID, "%s: last dimension must be contiguous", name);
    for (int d = 0; d < ndim - 1; ++d)
        if (t->stride[d] < 0) return fail(DSV4_ERR_INVALID, "%s: negative stride", name);
    return DSV4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct PoolInfo {
    bool fp8;
    int64_t pages;
    int64_t row_bytes;
};

dsv4_status check_pool(const char* name, const dsv4_tensor* t, PoolInfo* info) {
    if (t == nullptr || t->data == nullptr) return fail(DSV4_ERR_INVALID, "%s: NULL", name);
    if (t->dtype == DSV4_BF16) {
        DSV4_TRY(check_tensor(name, t, DSV4_BF16, 2, {-1, DSV4_HEAD_DIM}));
        if (t->stride[0] < DSV4_HEAD_DIM || t->stride[0] % 8 != 0)
            return fail(DSV4_ERR_INVALID, "%s: row stride must be >= 512 and a multiple of 8", name);
        if (!aligned16(t->data)) return fail(DSV4_ERR_INVALID, "%s: data must be 16-byte aligned", name);
        info->fp8 = false;
        info->pages = t->shape[0] / DSV4_PAGE_SIZE;
        info->row_bytes = t->stride[0] * 2;
        return DSV4_OK;
    }
    if (t->dtype == DSV4_U8) {
        DSV4_TRY(check_tensor(name, t, DSV4_U8, 2, {-1, DSV4_FP8_PAGE_BYTES}));
        if (t->stride[0] != DSV4_FP8_PAGE_BYTES)
            return fail(DSV4_ERR_INVALID, "%s: packed FP8 pages must be contiguous", name);
        if (!aligned16(t->data)) return fail(DSV4_ERR_INVALID, "%s: data must be 16-byte aligned", name);
        info->fp8 = true;
        info->pages = t->shape[0];
        info->row_bytes = 0;
        return DSV4_OK;
    }
    return fail(DSV4_ERR_INVALID, "%s: pool dtype must be bf16 rows or u8 packed FP8 pages", name);
}

struct Metadata {
    int32_t B = 0, T = 0, R = 0, W = 0, K = 0, P_swa = 0, P_extra = 0;
    Meta m{};
};

dsv4_status check_metadata(const dsv4_tensor* swa_page_table, const dsv4_tensor* extra_page_table,
                           const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens, const dsv4_tensor* qo_indptr,
                           int32_t T, int32_t compress_ratio, int32_t window, Metadata* md) {
    if (compress_ratio != 0 && compress_ratio != 4 && compress_ratio != 128)
        return fail(DSV4_ERR_UNSUPPORTED, "invalid compress_ratio %d (must be 0, 4 or 128)", compress_ratio);
    if (window < 1) return fail(DSV4_ERR_INVALID, "window must be >= 1 (got %d)", window);
    if (window > (1 << 20)) return fail(DSV4_ERR_UNSUPPORTED, "window %d above 2^20", window);
    DSV4_TRY(check_tensor("seq_lens", seq_lens, DSV4_I32, 1, {-1}));
    const int64_t B = seq_lens->shape[0];
    if (B < 1) return fail(DSV4_ERR_INVALID, "seq_lens: batch must be >= 1");
    DSV4_TRY(check_tensor("qo_indptr", qo_indptr, DSV4_I32, 1, {B + 1}));
    DSV4_TRY(check_tensor("swa_page_table", swa_page_table, DSV4_I32, 2, {B, -1}));
    if (swa_page_table->shape[1] < 1) return fail(DSV4_ERR_INVALID, "swa_page_table: needs >= 1 page per request");
    md->B = (int32_t)B;
    md->T = T;
    md->R = compress_ratio;
    md->W = window;
    md->P_swa = (int32_t)swa_page_table->shape[1];
    md->m.seq_lens = (const int32_t*)seq_lens->data;
    md->m.qo_indptr = (const int32_t*)qo_indptr->data;
    md->m.swa_table = (const int32_t*)swa_page_table->data;
    md->m.swa_ld = swa_page_table->stride[0];
    md->m.B = (int32_t)B;
    md->m.R = compress_ratio;
    md->m.W = window;
    if (compress_ratio != 0) {
        DSV4_TRY(check_tensor("extra_page_table", extra_page_table, DSV4_I32, 2, {B, -1}));
        if (extra_page_table->shape[1] < 1)
            return fail(DSV4_ERR_INVALID, "extra_page_table: needs >= 1 page per request");
        if (extra_page_table->shape[1] > (1 << 22) / DSV4_PAGE_SIZE * 64)
            return fail(DSV4_ERR_UNSUPPORTED, "extra_page_table: too many pages per request");
        md->P_extra = (int32_t)extra_page_table->shape[1];
        md->m.ext_table = (const int32_t*)extra_page_table->data;
        md->m.ext_ld = extra_page_table->stride[0];
    }
    if (compress_ratio == 4) {
        DSV4_TRY(check_tensor("c4_indices", c4_indices, DSV4_I32, 2, {T, -1}));
        if (c4_indices->shape[1] < 1) return fail(DSV4_ERR_INVALID, "c4_indices: width must be >= 1");
        if (c4_indices->shape[1] > (1 << 16)) return fail(DSV4_ERR_UNSUPPORTED, "c4_indices: width above 65536");
        md->K = (int32_t)c4_indices->shape[1];
        md->m.c4 = (const int32_t*)c4_indices->data;
        md->m.c4_ld = c4_indices->stride[0];
        md->m.K = md->K;
    }
    return DSV4_OK;
}

int64_t extra_bound(int32_t R, int32_t K, int32_t P_extra) {
    return R == 4 ? K : (R == 128 ? (int64_t)P_extra * DSV4_PAGE_SIZE : 0);
}

// ---- device properties and workspace ---------------------------------------

struct DeviceState {
    int cus = 0;
    void* ws = nullptr;  // split partials
    size_t ws_bytes = 0;
    // Buffers replaced by a larger one.  A HIP graph captured earlier may
    // still write into them, so they live until dsv4_attn_workspace_release.
    std::vector<void*> retired;
    const void* zero_row = nullptr;  // device address of g_zero_row
    void* scratch = nullptr;         // device address of `scratch`
    uint32_t* topk_count = nullptr;  // per-row counter and flag of the long-row top-k path, zero between calls
};
constexpr int kTopkMaxRowsSplit = 65535;  // rows of a long-row top-k call (grid y)
std::mutex g_mu;
std::vector<DeviceState> g_dev;
int32_t g_force_split_keys = 0;
int32_t g_force_kernel = DSV4_KERNEL_AUTO;  // 1..4 apply to bf16 pools, 5..6 to FP8 pools
// Test hook: key recording (dsv4_attn_debug_keys).
uint64_t* g_dbg_keys = nullptr;
int64_t g_dbg_keys_cap = 0;
uint32_t* g_dbg_masks = nullptr;
int64_t g_dbg_masks_cap = 0;

DeviceState* device_state(int dev) {
    if (dev < 0) return nullptr;
    if ((size_t)dev >= g_dev.size()) g_dev.resize(dev + 1);
    DeviceState& d = g_dev[dev];
    if (d.cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        d.cus = n;
    }
    return &d;
}

bool stream_capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return false;
    return cs != hipStreamCaptureStatusNone;
}

dsv4_status ensure_zero_row(DeviceState* d) {
    if (d->zero_row != nullptr) return DSV4_OK;
    void* p = nullptr;
    DSV4_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(g_zero_row)));
    d->zero_row = p;
    return DSV4_OK;
}

// The long-row top-k counters: allocated and zeroed once per device (outside
// any capture); every call leaves them at zero.
dsv4_status ensure_topk_count(DeviceState* d, hipStream_t st) {
    if (d->topk_count != nullptr) return DSV4_OK;
    if (stream_capturing(st))
        return fail(DSV4_ERR_WORKSPACE, "the top-k counters are not set up and the stream is being captured; call "
                                        "dsv4_attn_workspace_reserve before capturing");
    void* p = nullptr;
    if (hipMalloc(&p, 4 * sizeof(uint32_t) * kTopkMaxRowsSplit) != hipSuccess)
        return fail(DSV4_ERR_WORKSPACE, "hipMalloc of the top-k counters failed");
    DSV4_HIP(hipMemset(p, 0, 4 * sizeof(uint32_t) * kTopkMaxRowsSplit));
    DSV4_HIP(hipDeviceSynchronize());
    d->topk_count = (uint32_t*)p;  // kept for the life of the process
    return DSV4_OK;
}

dsv4_status ensure_scratch(DeviceState* d) {
    if (d->scratch != nullptr) return DSV4_OK;
    void* p = nullptr;
    DSV4_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    d->scratch = p;
    return DSV4_OK;
}

// Grows the workspace to at least `bytes` (at least doubling, so that a
// growing sequence of calls allocates O(log) times).  A call made while its
// stream is being captured never allocates: hipMalloc is not a stream
// operation and would break or escape the capture.
dsv4_status ensure_workspace(DeviceState* d, size_t bytes, hipStream_t st) {
    if (d->ws_bytes >= bytes) return DSV4_OK;
    if (stream_capturing(st))
        return fail(DSV4_ERR_WORKSPACE,
                    "the call needs %zu workspace bytes but %zu are reserved, and the stream is being captured; "
                    "call dsv4_attn_workspace_reserve with the largest size before capturing",
                    bytes, d->ws_bytes);
    size_t want = std::max({bytes, (size_t)16 << 20, 2 * d->ws_bytes});
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) return fail(DSV4_ERR_WORKSPACE, "hipMalloc of %zu workspace bytes failed", want);
    if (d->ws != nullptr) d->retired.push_back(d->ws);
    d->ws = p;
    d->ws_bytes = want;
    return DSV4_OK;
}

void plan_splits(int cus, int32_t T, int32_t H, int64_t nmax, Layout layout, int32_t* splits, int32_t* chunk);

// Kernel layout.  FP8 pools: the FP8 variant forced by dsv4_attn_set_kernel,
// else the 32-head one when there are at most 32 heads, or when its whole
// grid (rows x head blocks x its splits) fits the compute units once with at
// most kFp8H32MaxTiles tiles per split: with few rows the 64-head grid leaves
// compute units idle, and halving each workgroup's heads halves its products
// and operand decodes per tile, which is most of its loop; else the 64-head
// one, which loads each tile once for all 64 heads.  Measured on MI355X (C4
// decode at 1M tokens, 640 keys per row, per step, 64-head vs 32-head):
// 8 rows 16.8 vs 14.5 us (10 splits each), 16 rows 18.3 vs 16.4 (10 / 7
// splits), 24 rows 20.7 vs 19.1 (10 / 5), 32 rows 21.3 vs 20.5 (7 / 4),
// 64 rows 27.3 vs 29.3 (4 / 2 splits: the 32-head splits hold 10 tiles).
// bf16 pools: the variant forced by dsv4_attn_set_kernel, else the 16-head
// kernel for at most 16 heads (no padding of heads); above that the 32-head
// score/PV role kernel while its whole grid (rows x 32-head blocks x its
// splits) needs less than two rounds of workgroups on the compute units,
// and the 64-head kernel, which loads each tile once for all 64 heads, from
// two rounds on (more than 32 heads; for
// 17-32 heads, only when the rows alone give every compute unit two 64-head
// workgroups, since a 64-head workgroup then multiplies padded heads).
// Measured on MI355X (graph replay per call, roles vs 64-head; the roles
// grid in rounds of 256 workgroups): C4 decode 32 rows 16.8 vs 17.1 us
// (32-head dim split), 128 rows (1 round) 29.1 vs 39.0, 160 rows (1.25)
// 48.7 vs 55.3, 192 rows (1.5) 53.9 vs 62.0, 256 rows (2) 62.7 vs 57.2; C128
// decode at 128K, 64 rows (1) 30.9 vs 33.2 us, 96 rows (1.5) 55.0 vs 56.6,
// 128 rows (2) 63.7 vs 55.4, 512 rows (8) 215 vs 188; C4 verify 128 rows
// (1) 28.6 vs 31.0 us, 192 rows (1.5) 50.4 vs 57.6, 512 rows (4) 108 vs 97;
// C4 prefill 4 x 2048 rows 1.28 vs 1.02 ms; C128 prefill 0.94 vs 0.74 ms.
Layout choose_layout(int32_t T, int32_t H, int cus, bool fp8, int64_t nmax) {
    if (fp8) {
        if (g_force_kernel == DSV4_KERNEL_FP8) return Layout::kFp8;
        if (g_force_kernel == DSV4_KERNEL_FP8_H32 || H <= kWide32HeadsPerBlock) return Layout::kFp8H32;
        constexpr int kFp8H32MaxTiles = 6;
        int32_t s = 1, c = 0;
        plan_splits(cus, T, H, nmax, Layout::kFp8H32, &s, &c);
        const int64_t items = (int64_t)T * ((H + kWide32HeadsPerBlock - 1) / kWide32HeadsPerBlock) * s;
        return items <= cus && c <= kFp8H32MaxTiles * kTileKeys ? Layout::kFp8H32 : Layout::kFp8;
    }
    switch (g_force_kernel) {
        case DSV4_KERNEL_H16: return Layout::kNarrow;
        case DSV4_KERNEL_H32: return Layout::kWide32;
        case DSV4_KERNEL_H32_ROLES: return Layout::kRoles32;
        case DSV4_KERNEL_H64: return Layout::kWide;
        default: break;
    }
    if (H <= kNarrowHeadsPerBlock) return Layout::kNarrow;
    if (H <= kWide32HeadsPerBlock) return (int64_t)T >= 2 * (int64_t)cus ? Layout::kWide : Layout::kRoles32;
    int32_t s = 1, c = 0;
    plan_splits(cus, T, H, nmax, Layout::kRoles32, &s, &c);
    const int64_t items = (int64_t)T * ((H + kWide32HeadsPerBlock - 1) / kWide32HeadsPerBlock) * s;
    return items < 2 * (int64_t)cus ? Layout::kRoles32 : Layout::kWide;
}

int32_t heads_per_block(Layout layout) {
    switch (layout) {
        case Layout::kWide32:
        case Layout::kRoles32:
        case Layout::kFp8H32: return kWide32HeadsPerBlock;
        case Layout::kNarrow: return kNarrowHeadsPerBlock;
        default: return kWideHeadsPerBlock;
    }
}

int32_t kernel_id(Layout layout) {
    switch (layout) {
        case Layout::kNarrow: return DSV4_KERNEL_H16;
        case Layout::kWide32: return DSV4_KERNEL_H32;
        case Layout::kRoles32: return DSV4_KERNEL_H32_ROLES;
        case Layout::kWide: return DSV4_KERNEL_H64;
        case Layout::kFp8H32: return DSV4_KERNEL_FP8_H32;
        default: return DSV4_KERNEL_FP8;
    }
}

// Keys per LDS tile and most keys per split of each split kernel.
int32_t tile_keys(Layout layout) { return layout == Layout::kNarrow ? kNarrowTileKeys : kTileKeys; }
int32_t max_split_keys(Layout layout) { return layout == Layout::kNarrow ? kNarrowMaxSplitKeys : kMaxSplitKeys; }

// Keys per split: enough splits per row to fill the chip once, with at
// least 64 keys (2 tiles) per split; for bf16 at least 128 keys (4 tiles)
// when that still occupies half the compute units, which spreads the fixed
// per-workgroup cost (metadata, Q, partial write) over more tiles.
// (Measured on MI355X, FP8 C4 decode at 1M tokens, 8 rows, per step:
// 20 splits of 32 keys 17.9 us, 10 of 64 17.0 us, 7 of 96 17.9 us; the
// shorter splits' extra partials and merge outweigh their shorter loop.)
void plan_splits(int cus, int32_t T, int32_t H, int64_t nmax, Layout layout, int32_t* splits, int32_t* chunk) {
    const bool fp8 = layout == Layout::kFp8 || layout == Layout::kFp8H32;
    const int64_t hpb = heads_per_block(layout);
    const int64_t head_blocks = (H + hpb - 1) / hpb;
    int64_t c;
    if (g_force_split_keys > 0) {
        c = g_force_split_keys;
    } else {
        const int64_t rows = std::max<int64_t>(1, (int64_t)T * head_blocks);
        int64_t want = (cus + rows - 1) / rows;  // splits per row to fill the chip once
        const int64_t min_keys = 64;
        const int64_t most = std::max<int64_t>(1, (nmax + min_keys - 1) / min_keys);
        want = std::min(std::max<int64_t>(want, 1), most);
        if (!fp8) {
            const int64_t w128 = std::min(want, std::max<int64_t>(1, (nmax + 127) / 128));
            if (rows * w128 * 2 >= cus) want = w128;
        }
        c = (nmax + want - 1) / want;
        const int64_t unit = tile_keys(layout);
        c = (c + unit - 1) / unit * unit;
        // When a workgroup's key limit forces more splits than wanted, make
        // them equal rather than leaving a short last one: the workgroups of
        // a call end together only if their splits are alike (measured:
        // C128 decode at 1152 keys per row, 128 requests, roles kernel:
        // 1024 + 128 keys 64.3 us against 53.2 us for 2 x 576 keys).
        if (c > max_split_keys(layout)) {
            const int64_t n = (nmax + max_split_keys(layout) - 1) / max_split_keys(layout);
            c = ((nmax + n - 1) / n + unit - 1) / unit * unit;
        }
    }
    c = (c + tile_keys(layout) - 1) / tile_keys(layout) * tile_keys(layout);
    c = std::min<int64_t>(std::max<int64_t>(c, tile_keys(layout)), max_split_keys(layout));
    *chunk = (int32_t)c;
    *splits = (int32_t)std::max<int64_t>(1, (nmax + c - 1) / c);
}

// ---- timing -------------------------------------------------------------------
// e0 before the split kernel, e1 between it and the merge kernel, e2 after
// the merge kernel (none when no row is split: there is no merge kernel).
struct TimingRec {
    hipEvent_t e0, e1, e2;
};
bool g_timing = false;
std::vector<TimingRec> g_timing_recs;
std::vector<hipEvent_t> g_event_pool;

// Inside stream capture a record becomes an event-record node appended to the
// captured graph after the stream's current dependencies, so each replay
// re-records it; reading after a replay gives that replay's times.  The null
// stream cannot be captured.
hipError_t record_event(hipEvent_t e, hipStream_t st) {
    if (st == nullptr) return hipEventRecord(e, st);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    hipGraph_t graph = nullptr;
    const hipGraphNode_t* deps = nullptr;
    size_t n_deps = 0;
    hipError_t err = hipStreamGetCaptureInfo_v2(st, &cs, &id, &graph, &deps, &n_deps);
    if (err != hipSuccess) return err;
    if (cs != hipStreamCaptureStatusActive) return hipEventRecord(e, st);
    hipGraphNode_t node = nullptr;
    err = hipGraphAddEventRecordNode(&node, graph, deps, n_deps, e);
    if (err != hipSuccess) return err;
    return hipStreamUpdateCaptureDependencies(st, &node, 1, hipStreamSetCaptureDependencies);
}

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    // Timing only: no system-scope fence when the event is recorded (such a
    // fence writes back and invalidates the caches, which would both stretch
    // the interval and slow the kernel that follows).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// ---- DSV4_VALIDATE: synchronous host check of device-resident contents ------
bool validate_enabled() {
    const char* v = getenv("DSV4_VALIDATE");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
}

template <typename T>
dsv4_status fetch(const dsv4_tensor* t, std::vector<T>& host, int64_t rows, int64_t cols) {
    host.assign((size_t)(rows * cols), T{});
    const int64_t ld = t->ndim == 2 ? t->stride[0] : cols;
    for (int64_t r = 0; r < rows; ++r)
        DSV4_HIP(hipMemcpy(host.data() + r * cols, (const T*)t->data + r * ld, sizeof(T) * cols, hipMemcpyDeviceToHost));
    return DSV4_OK;
}

dsv4_status validate_contents(const Metadata& md, const dsv4_tensor* swa_page_table,
                              const dsv4_tensor* extra_page_table, const dsv4_tensor* c4_indices,
                              const dsv4_tensor* seq_lens, const dsv4_tensor* qo_indptr, int64_t swa_pages,
                              int64_t extra_pages, hipStream_t stream) {
    DSV4_HIP(hipStreamSynchronize(stream));
    std::vector<int32_t> sl, qo, st, et, c4;
    DSV4_TRY(fetch(seq_lens, sl, 1, md.B));
    DSV4_TRY(fetch(qo_indptr, qo, 1, md.B + 1));
    DSV4_TRY(fetch(swa_page_table, st, md.B, md.P_swa));
    if (md.R) DSV4_TRY(fetch(extra_page_table, et, md.B, md.P_extra));
    if (md.R == 4) DSV4_TRY(fetch(c4_indices, c4, md.T, md.K));
    if (qo[0] != 0) return fail(DSV4_ERR_CONTRACT, "qo_indptr[0] = %d, expected 0", qo[0]);
    for (int r = 0; r < md.B; ++r)
        if (qo[r + 1] < qo[r]) return fail(DSV4_ERR_CONTRACT, "qo_indptr decreases at %d", r);
    if (qo[md.B] != md.T) return fail(DSV4_ERR_CONTRACT, "qo_indptr[B] = %d, expected T = %d", qo[md.B], md.T);
    auto page_ok = [](const std::vector<int32_t>& tab, int64_t ld, int r, int64_t x, int64_t pages) {
        const int64_t lp = x / DSV4_PAGE_SIZE;
        if (lp >= ld) return false;
        const int32_t pg = tab[(size_t)(r * ld + lp)];
        return pg >= 0 && pg < pages;
    };
    for (int r = 0; r < md.B; ++r) {
        const int64_t nq = qo[r + 1] - qo[r];
        if (nq > sl[r]) return fail(DSV4_ERR_CONTRACT, "request %d: %lld rows but seq_len %d", r, (long long)nq, sl[r]);
        for (int64_t t = qo[r]; t < qo[r + 1]; ++t) {
            const int64_t p = sl[r] - nq + (t - qo[r]);
            const int64_t lo = std::max<int64_t>(0, p - md.W + 1);
            if (p < 0) return fail(DSV4_ERR_CONTRACT, "row %lld: negative position", (long long)t);
            for (int64_t lp = lo / DSV4_PAGE_SIZE; lp <= p / DSV4_PAGE_SIZE; ++lp)
                if (!page_ok(st, md.P_swa, r, lp * DSV4_PAGE_SIZE, swa_pages))
                    return fail(DSV4_ERR_CONTRACT, "row %lld: SWA page %lld is not mapped", (long long)t,
                                (long long)lp);
            const int64_t vis = md.R ? (p + 1) / md.R : 0;
            if (md.R == 4) {
                for (int k = 0; k < md.K; ++k) {
                    const int64_t c = c4[(size_t)(t * md.K + k)];
                    if (c < -1 || c >= vis)
                        return fail(DSV4_ERR_CONTRACT, "row %lld: C4 index %lld outside [-1, %lld)", (long long)t,
                                    (long long)c, (long long)vis);
                    if (c >= 0 && !page_ok(et, md.P_extra, r, c, extra_pages))
                        return fail(DSV4_ERR_CONTRACT, "row %lld: C4 entry %lld has no page", (long long)t,
                                    (long long)c);
                }
            } else if (md.R == 128) {
                for (int64_t lp = 0; lp * DSV4_PAGE_SIZE < vis; ++lp)
                    if (!page_ok(et, md.P_extra, r, lp * DSV4_PAGE_SIZE, extra_pages))
                        return fail(DSV4_ERR_CONTRACT, "row %lld: C128 page %lld is not mapped", (long long)t,
                                    (long long)lp);
            }
        }
    }
    return DSV4_OK;
}

}  // namespace

extern "C" {

const char* dsv4_last_error(void) { return g_err.c_str(); }

int32_t dsv4_abi_version(void) { return DSV4_ABI_VERSION; }

dsv4_status dsv4_attn_set_split_keys(int32_t keys_per_split) {
    if (keys_per_split < 0 || keys_per_split % kNarrowTileKeys != 0 || keys_per_split > kNarrowMaxSplitKeys)
        return fail(DSV4_ERR_INVALID, "keys_per_split must be 0 or a multiple of %d up to %d", kNarrowTileKeys,
                    kNarrowMaxSplitKeys);
    std::lock_guard<std::mutex> lk(g_mu);
    g_force_split_keys = keys_per_split;
    return DSV4_OK;
}

dsv4_status dsv4_attn_set_kernel(int32_t kernel) {
    if (kernel < DSV4_KERNEL_AUTO || kernel > DSV4_KERNEL_FP8_H32)
        return fail(DSV4_ERR_INVALID, "kernel must be DSV4_KERNEL_AUTO (0) or a split-kernel variant (1..6), got %d",
                    kernel);
    std::lock_guard<std::mutex> lk(g_mu);
    g_force_kernel = kernel;
    return DSV4_OK;
}

dsv4_status dsv4_attn_plan(int32_t num_rows, int32_t num_heads, int32_t compress_ratio, int32_t window,
                           int32_t c4_width, int32_t extra_pages, int32_t kv_fp8, int32_t* splits,
                           int32_t* keys_per_split, int32_t* kernel) {
    if (splits == nullptr || keys_per_split == nullptr) return fail(DSV4_ERR_INVALID, "NULL output");
    if (compress_ratio != 0 && compress_ratio != 4 && compress_ratio != 128)
        return fail(DSV4_ERR_UNSUPPORTED, "invalid compress_ratio %d (must be 0, 4 or 128)", compress_ratio);
    if (num_rows < 0 || num_heads < 1 || num_heads > 128 || window < 1)
        return fail(DSV4_ERR_INVALID, "bad sizes");
    int dev = 0;
    int cus = 256;
    std::lock_guard<std::mutex> lk(g_mu);
    if (hipGetDevice(&dev) == hipSuccess) {
        DeviceState* d = device_state(dev);
        if (d) cus = d->cus;
    }
    const int64_t nmax = (int64_t)window + extra_bound(compress_ratio, c4_width, extra_pages);
    const Layout layout = choose_layout(num_rows, num_heads, cus, kv_fp8 != 0, nmax);
    plan_splits(cus, num_rows, num_heads, nmax, layout, splits, keys_per_split);
    if (kernel != nullptr) *kernel = kernel_id(layout);
    return DSV4_OK;
}

dsv4_status dsv4_attn_workspace_reserve(size_t bytes, void* stream) {
    int dev = 0;
    DSV4_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState* d = device_state(dev);
    DSV4_TRY(ensure_zero_row(d));
    DSV4_TRY(ensure_topk_count(d, (hipStream_t)stream));
    return ensure_workspace(d, bytes, (hipStream_t)stream);
}

void dsv4_attn_workspace_release(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (size_t i = 0; i < g_dev.size(); ++i) {
        DeviceState& d = g_dev[i];
        if (d.ws == nullptr && d.retired.empty()) continue;
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice((int)i) == hipSuccess) {
            (void)hipDeviceSynchronize();
            if (d.ws != nullptr) (void)hipFree(d.ws);
            for (void* p : d.retired) (void)hipFree(p);
            (void)hipSetDevice(cur);
        }
        d.ws = nullptr;
        d.ws_bytes = 0;
        d.retired.clear();
    }
}

dsv4_status dsv4_attn_debug_keys(void* keys, int64_t keys_cap, void* masks, int64_t masks_cap) {
    if (keys != nullptr && (keys_cap < 0 || masks == nullptr || masks_cap < 0))
        return fail(DSV4_ERR_INVALID, "debug keys: need both buffers and non-negative capacities");
    std::lock_guard<std::mutex> lk(g_mu);
    g_dbg_keys = (uint64_t*)keys;
    g_dbg_keys_cap = keys ? keys_cap : 0;
    g_dbg_masks = keys ? (uint32_t*)masks : nullptr;
    g_dbg_masks_cap = keys ? masks_cap : 0;
    return DSV4_OK;
}

dsv4_status dsv4_attn_timing_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_timing = enable != 0;
    return DSV4_OK;
}

dsv4_status dsv4_attn_timing_read(double* split_ms, double* merge_ms, int64_t* calls) {
    std::lock_guard<std::mutex> lk(g_mu);
    double a = 0.0, b = 0.0;
    for (TimingRec& r : g_timing_recs) {
        DSV4_HIP(hipEventSynchronize(r.e2 != nullptr ? r.e2 : r.e1));
        float x = 0.f, y = 0.f;
        DSV4_HIP(hipEventElapsedTime(&x, r.e0, r.e1));
        if (r.e2 != nullptr) DSV4_HIP(hipEventElapsedTime(&y, r.e1, r.e2));
        a += x;
        b += y;
        g_event_pool.push_back(r.e0);
        g_event_pool.push_back(r.e1);
        if (r.e2 != nullptr) g_event_pool.push_back(r.e2);
    }
    if (calls) *calls = (int64_t)g_timing_recs.size();
    g_timing_recs.clear();
    if (split_ms) *split_ms = a;
    if (merge_ms) *merge_ms = b;
    return DSV4_OK;
}

dsv4_status dsv4_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return fail(DSV4_ERR_INVALID, "bytes must be a nonnegative multiple of 16, got %lld", (long long)bytes);
    if (workgroups < 1 || workgroups > (1 << 20))
        return fail(DSV4_ERR_INVALID, "workgroups must be 1 .. 2^20, got %d", workgroups);
    if (bytes == 0) return DSV4_OK;
    if (buf == nullptr || !aligned16(buf)) return fail(DSV4_ERR_INVALID, "buf must be a 16-byte aligned device pointer");
    if (sink == nullptr || !aligned16(sink)) return fail(DSV4_ERR_INVALID, "sink must be a 16-byte aligned device pointer");
    DSV4_HIP(launch_read_probe(buf, bytes, workgroups, sink, (hipStream_t)stream));
    return DSV4_OK;
}

dsv4_status dsv4_attn_gather_slots(const dsv4_tensor* swa_page_table, const dsv4_tensor* extra_page_table,
                                   const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens,
                                   const dsv4_tensor* qo_indptr, int32_t num_rows, int32_t compress_ratio,
                                   int32_t window, const dsv4_tensor* slots, const dsv4_tensor* counts,
                                   void* stream) {
    if (num_rows < 0) return fail(DSV4_ERR_INVALID, "num_rows must be >= 0");
    Metadata md;
    DSV4_TRY(check_metadata(swa_page_table, extra_page_table, c4_indices, seq_lens, qo_indptr, num_rows,
                            compress_ratio, window, &md));
    const int64_t need = (int64_t)window + extra_bound(md.R, md.K, md.P_extra);
    DSV4_TRY(check_tensor("slots", slots, DSV4_I32, 2, {num_rows, -1}));
    if (slots->shape[1] < need)
        return fail(DSV4_ERR_INVALID, "slots: width %lld below window + extra bound %lld", (long long)slots->shape[1],
                    (long long)need);
    DSV4_TRY(check_tensor("counts", counts, DSV4_I32, 2, {num_rows, 2}));
    if (counts->stride[0] != 2) return fail(DSV4_ERR_INVALID, "counts must be contiguous");
    if (num_rows == 0) return DSV4_OK;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled())
        DSV4_TRY(validate_contents(md, swa_page_table, extra_page_table, c4_indices, seq_lens, qo_indptr,
                                   INT64_MAX, INT64_MAX, st));
    GatherArgs g{};
    g.m = md.m;
    g.T = num_rows;
    g.slots = (int32_t*)slots->data;
    g.slots_ld = slots->stride[0];
    g.counts = (int32_t*)counts->data;
    if (g.slots_ld < slots->shape[1]) return fail(DSV4_ERR_INVALID, "slots: rows overlap");
    DSV4_HIP(launch_gather(g, st));
    return DSV4_OK;
}

dsv4_status dsv4_kv_pack_fp8(const dsv4_tensor* k, const dsv4_tensor* slots, const dsv4_tensor* pool, void* stream) {
    DSV4_TRY(check_tensor("k", k, DSV4_BF16, 2, {-1, DSV4_HEAD_DIM}));
    const int64_t n = k->shape[0];
    DSV4_TRY(check_tensor("slots", slots, DSV4_I32, 1, {n}));
    PoolInfo pi{};
    DSV4_TRY(check_pool("pool", pool, &pi));
    if (!pi.fp8) return fail(DSV4_ERR_UNSUPPORTED, "pool: the FP8 store needs a packed FP8 pool (u8 pages)");
    if (n == 0) return DSV4_OK;
    if (k->stride[0] % 8 != 0 || !aligned16(k->data))
        return fail(DSV4_ERR_INVALID, "k: rows must be 16-byte aligned (row stride a multiple of 8)");
    if (n > 1 && k->stride[0] < DSV4_HEAD_DIM) return fail(DSV4_ERR_INVALID, "k: rows overlap");
    if (pi.pages < 1) return fail(DSV4_ERR_INVALID, "pool: no pages");
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        DSV4_HIP(hipStreamSynchronize(st));
        std::vector<int32_t> host;
        DSV4_TRY(fetch(slots, host, 1, n));
        std::vector<int32_t> seen;
        for (int64_t i = 0; i < n; ++i) {
            if (host[i] < 0) continue;
            if ((int64_t)host[i] >= pi.pages * DSV4_PAGE_SIZE)
                return fail(DSV4_ERR_CONTRACT, "slots[%lld] = %d beyond the pool's %lld slots", (long long)i, host[i],
                            (long long)(pi.pages * DSV4_PAGE_SIZE));
            seen.push_back(host[i]);
        }
        std::sort(seen.begin(), seen.end());
        if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
            return fail(DSV4_ERR_CONTRACT, "slots: a slot appears twice");
    }
    PackArgs p{};
    p.k = (const uint16_t*)k->data;
    p.k_s0 = k->stride[0];
    p.slots = (const int32_t*)slots->data;
    p.n = n;
    p.pool = (uint8_t*)pool->data;
    p.page_bytes = DSV4_FP8_PAGE_BYTES;
    DSV4_HIP(launch_pack_fp8(p, st));
    return DSV4_OK;
}

dsv4_status dsv4_c4_topk(const dsv4_tensor* scores, const dsv4_tensor* num_candidates, const dsv4_tensor* indices,
                         void* stream) {
    DSV4_TRY(check_tensor("scores", scores, DSV4_F32, 2, {-1, -1}));
    const int64_t T = scores->shape[0], ld = scores->shape[1];
    DSV4_TRY(check_tensor("num_candidates", num_candidates, DSV4_I32, 1, {T}));
    DSV4_TRY(check_tensor("indices", indices, DSV4_I32, 2, {T, -1}));
    const int64_t K = indices->shape[1];
    if (K < 1 || K > kTopkMaxK) return fail(DSV4_ERR_UNSUPPORTED, "indices: width %lld, expected 1..%d", (long long)K, kTopkMaxK);
    if (T > INT32_MAX || ld > INT32_MAX) return fail(DSV4_ERR_UNSUPPORTED, "scores: too large");
    if (T == 0) return DSV4_OK;
    if (T > 1 && indices->stride[0] < K) return fail(DSV4_ERR_INVALID, "indices: rows overlap");
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        DSV4_HIP(hipStreamSynchronize(st));
        std::vector<int32_t> host;
        DSV4_TRY(fetch(num_candidates, host, 1, T));
        for (int64_t t = 0; t < T; ++t)
            if (host[t] < 0 || host[t] > ld)
                return fail(DSV4_ERR_CONTRACT, "num_candidates[%lld] = %d outside 0..%lld", (long long)t, host[t],
                            (long long)ld);
    }
    TopkArgs a{};
    a.scores = (const float*)scores->data;
    a.s_ld = scores->stride[0];
    a.n_cand = (const int32_t*)num_candidates->data;
    a.out = (int32_t*)indices->data;
    a.out_ld = indices->stride[0];
    a.T = (int32_t)T;
    a.K = (int32_t)K;
    a.ld = (int32_t)ld;
    const size_t ws_bytes = T <= kTopkMaxRowsSplit ? topk_workspace_bytes(T, ld, K) : 0;
    int dev = 0;
    DSV4_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_mu);
    if (ws_bytes > 0) {  // long rows: several workgroups per row, survivor lists in the workspace
        DeviceState* d = device_state(dev);
        DSV4_TRY(ensure_topk_count(d, st));
        DSV4_TRY(ensure_workspace(d, ws_bytes, st));
        topk_bind_workspace(a, d->ws, d->topk_count);
    }
    DSV4_HIP(launch_topk(a, st));
    return DSV4_OK;
}

}  // extern "C"

namespace {

// Both forward entry points.  noalloc: split partials go to the static
// `scratch` array (calls whose partials do not fit are refused) and the
// timing hook is ignored (its events would be created on demand).
dsv4_status forward_impl(const dsv4_tensor* q, const dsv4_tensor* swa_pool, const dsv4_tensor* swa_page_table,
                         const dsv4_tensor* extra_pool, const dsv4_tensor* extra_page_table,
                         const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens, const dsv4_tensor* qo_indptr,
                         const dsv4_tensor* sink, int32_t compress_ratio, int32_t window, float scale,
                         const dsv4_tensor* out, const dsv4_tensor* lse, void* stream, bool noalloc) {
    if (q == nullptr) return fail(DSV4_ERR_INVALID, "q: NULL descriptor");
    DSV4_TRY(check_tensor("q", q, DSV4_BF16, 3, {-1, -1, DSV4_HEAD_DIM}));
    const int64_t T = q->shape[0], H = q->shape[1];
    if (q->stride[1] != 0 && H > 1 && q->stride[1] < DSV4_HEAD_DIM) return fail(DSV4_ERR_INVALID, "q: heads overlap");
    if (H < 1 || H > 128) return fail(DSV4_ERR_INVALID, "q: %lld heads, expected 1..128", (long long)H);
    if (T > (1 << 24)) return fail(DSV4_ERR_UNSUPPORTED, "q: more than 2^24 rows");
    if (T > 0 && (q->stride[0] % 8 || q->stride[1] % 8 || !aligned16(q->data)))
        return fail(DSV4_ERR_INVALID, "q: rows must be 16-byte aligned (strides multiple of 8)");
    if (!std::isfinite(scale)) return fail(DSV4_ERR_INVALID, "scale must be finite");

    Metadata md;
    DSV4_TRY(check_metadata(swa_page_table, extra_page_table, c4_indices, seq_lens, qo_indptr, (int32_t)T,
                            compress_ratio, window, &md));
    PoolInfo swa{}, ext{};
    DSV4_TRY(check_pool("swa_pool", swa_pool, &swa));
    if (compress_ratio != 0) {
        DSV4_TRY(check_pool("extra_pool", extra_pool, &ext));
        if (ext.fp8 != swa.fp8)
            return fail(DSV4_ERR_UNSUPPORTED, "swa_pool and extra_pool must use the same KV format");
    }
    if (sink != nullptr) DSV4_TRY(check_tensor("sink", sink, DSV4_F32, 1, {H}));
    DSV4_TRY(check_tensor("out", out, DSV4_BF16, 3, {T, H, DSV4_HEAD_DIM}));
    if (T > 0 && (out->stride[0] % 4 || out->stride[1] % 4 || (reinterpret_cast<uintptr_t>(out->data) & 7u)))
        return fail(DSV4_ERR_INVALID, "out: rows must be 8-byte aligned (strides multiple of 4)");
    if (lse != nullptr) DSV4_TRY(check_tensor("lse", lse, DSV4_F32, 2, {T, H}));
    if (T == 0) return DSV4_OK;

    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled())
        DSV4_TRY(validate_contents(md, swa_page_table, extra_page_table, c4_indices, seq_lens, qo_indptr, swa.pages,
                                   compress_ratio ? ext.pages : 0, st));

    int dev = 0;
    DSV4_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState* d = device_state(dev);
    DSV4_TRY(ensure_zero_row(d));

    AttnArgs a{};
    a.zero_row = (const uint8_t*)d->zero_row;
    a.m = md.m;
    a.q = (const uint16_t*)q->data;
    a.q_s0 = q->stride[0];
    a.q_s1 = q->stride[1];
    a.swa_pool = (const uint8_t*)swa_pool->data;
    a.swa_row_bytes = swa.row_bytes;
    a.ext_pool = compress_ratio ? (const uint8_t*)extra_pool->data : a.swa_pool;
    a.ext_row_bytes = compress_ratio ? ext.row_bytes : swa.row_bytes;
    a.sink = sink ? (const float*)sink->data : nullptr;
    a.T = (int32_t)T;
    a.H = (int32_t)H;
    a.scale_log2 = scale * 1.4426950408889634f;
    const int64_t nmax = (int64_t)window + extra_bound(md.R, md.K, md.P_extra);
    const Layout layout = choose_layout(a.T, a.H, d->cus, swa.fp8, nmax);
    plan_splits(d->cus, a.T, a.H, nmax, layout, &a.splits, &a.chunk);
    a.head_blocks = (int32_t)((H + heads_per_block(layout) - 1) / heads_per_block(layout));
    a.ext_pages = md.P_extra;
    const int64_t n_items = (int64_t)a.T * a.head_blocks * a.splits;
    if (n_items > (int64_t)1 << 30) return fail(DSV4_ERR_UNSUPPORTED, "too many work items (%lld)", (long long)n_items);
    a.n_items = (int32_t)n_items;
    a.out = (uint16_t*)out->data;
    a.out_s0 = out->stride[0];
    a.out_s1 = out->stride[1];
    a.lse = lse ? (float*)lse->data : nullptr;
    a.lse_s0 = lse ? lse->stride[0] : 0;
    if (a.splits > 1) {
        const size_t n_part = (size_t)T * a.splits * H;
        const size_t bytes_o = n_part * DSV4_HEAD_DIM * sizeof(uint16_t);
        const size_t need = bytes_o + n_part * sizeof(float);
        void* ws = nullptr;
        if (noalloc) {
            if (need > kScratchBytes)
                return fail(DSV4_ERR_WORKSPACE,
                            "the call's split partials need %zu bytes, above the %zu-byte static scratch of the "
                            "no-allocation entry point (T x splits x H x 1028 bytes)",
                            need, kScratchBytes);
            DSV4_TRY(ensure_scratch(d));
            ws = d->scratch;
        } else {
            DSV4_TRY(ensure_workspace(d, need, st));
            ws = d->ws;
        }
        a.ws_o = (uint16_t*)ws;
        a.ws_lse = (float*)((char*)ws + bytes_o);
    }

    if (g_dbg_keys != nullptr) {
        const int64_t units = (int64_t)a.T * a.head_blocks * a.splits;
        if (units * a.chunk > g_dbg_keys_cap || units * 32 > g_dbg_masks_cap)
            return fail(DSV4_ERR_INVALID, "debug keys: buffers hold %lld / %lld entries, the call needs %lld / %lld",
                        (long long)g_dbg_keys_cap, (long long)g_dbg_masks_cap, (long long)(units * a.chunk),
                        (long long)(units * 32));
        a.dbg_keys = g_dbg_keys;
        a.dbg_masks = g_dbg_masks;
    }

    TimingRec rec{};
    const bool timing = g_timing && !noalloc;
    if (timing) {
        rec.e0 = take_event();
        rec.e1 = take_event();
        rec.e2 = a.splits > 1 ? take_event() : nullptr;  // no merge kernel: no interval to time
        if (!rec.e0 || !rec.e1 || (a.splits > 1 && !rec.e2)) return fail(DSV4_ERR_HIP, "hipEventCreate failed");
        DSV4_HIP(record_event(rec.e0, st));
    }
    DSV4_HIP(launch_attention(a, layout, st));
    if (timing) DSV4_HIP(record_event(rec.e1, st));
    if (a.splits > 1) DSV4_HIP(launch_merge(a, st));
    if (timing) {
        if (rec.e2 != nullptr) DSV4_HIP(record_event(rec.e2, st));
        g_timing_recs.push_back(rec);
    }
    return DSV4_OK;
}

}  // namespace

extern "C" {

dsv4_status dsv4_attn_forward(const dsv4_tensor* q, const dsv4_tensor* swa_pool, const dsv4_tensor* swa_page_table,
                              const dsv4_tensor* extra_pool, const dsv4_tensor* extra_page_table,
                              const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens,
                              const dsv4_tensor* qo_indptr, const dsv4_tensor* sink, int32_t compress_ratio,
                              int32_t window, float scale, const dsv4_tensor* out, const dsv4_tensor* lse,
                              void* stream) {
    return forward_impl(q, swa_pool, swa_page_table, extra_pool, extra_page_table, c4_indices, seq_lens, qo_indptr,
                        sink, compress_ratio, window, scale, out, lse, stream, false);
}

dsv4_status dsv4_attn_forward_noalloc(const dsv4_tensor* q, const dsv4_tensor* swa_pool,
                                      const dsv4_tensor* swa_page_table, const dsv4_tensor* extra_pool,
                                      const dsv4_tensor* extra_page_table, const dsv4_tensor* c4_indices,
                                      const dsv4_tensor* seq_lens, const dsv4_tensor* qo_indptr,
                                      const dsv4_tensor* sink, int32_t compress_ratio, int32_t window, float scale,
                                      const dsv4_tensor* out, const dsv4_tensor* lse, void* stream) {
    return forward_impl(q, swa_pool, swa_page_table, extra_pool, extra_page_table, c4_indices, seq_lens, qo_indptr,
                        sink, compress_ratio, window, scale, out, lse, stream, true);
}

size_t dsv4_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
