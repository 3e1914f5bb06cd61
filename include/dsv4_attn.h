/*
 * dsv4_attn.h -- C ABI of the MI355X (gfx950) DeepSeek-V4 hybrid sparse MQA
 * attention library, decode and target-verify.
 *
 * The operation (sources: "SGLang DeepSeek-V4 attention test capability
 * matrix" page; "DeepSeek-V4 Attention: Query, cache write and history
 * addressing" page; the Day-0 overview page, section "what V4 changed"):
 *
 *   Query row t of request r sits at position p = seq_lens[r] - n_q + (t -
 *   qo_indptr[r]), n_q = qo_indptr[r+1] - qo_indptr[r] (walk-through, sections
 *   1 and 4).  Its keys are the sliding window x = max(0, p-W+1) .. p of the
 *   SWA cache, followed by, for compress_ratio R (overview "hybrid sparse
 *   attention"; walk-through section 5):
 *     R = 0   -- nothing;
 *     R = 4   -- the C4 entries named by c4_indices[t][0..K-1] (-1 = none),
 *                every named entry must be visible: 0 <= c < (p+1)/4;
 *     R = 128 -- every visible C128 entry c = 0 .. (p+1)/128 - 1.
 *   Logical position x (token or compressed entry) of request r lives in slot
 *   table[r][x / 256] * 256 + x % 256 of its pool (page size 256, asserted by
 *   the test-matrix page).  One KV head serves all H query heads and the value
 *   of a key is the key row itself (V = K, walk-through section 3).  A per-head
 *   sink logit joins the softmax as a virtual key with value zero (test-matrix
 *   page, "attention-sink correction"); it is NOT multiplied by `scale`:
 *
 *     s_k   = scale * <q[t,h,:], K_k>
 *     out   = sum_k e^{s_k} K_k / (sum_k e^{s_k} + e^{sink[h]})
 *     lse   = ln(sum_k e^{s_k} + e^{sink[h]})          (natural log)
 *
 * Head geometry: 512 = 448 non-rotary + 64 rotary dims (test-matrix page,
 * "input and config coverage"); Q arrives with RoPE applied, and the output
 * keeps the rotary dims (inverse RoPE comes after attention).
 *
 * Conventions for every entry point:
 *  - Tensors are non-owning descriptors; the caller keeps ownership of all
 *    memory and of the stream.  No pointer is retained after return.
 *  - Device pointers unless stated.  Shapes/strides are in elements; the last
 *    dimension must be contiguous (stride 1).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *    The host never reads device memory, so seq_lens, qo_indptr, page tables
 *    and indices may change between calls without a host sync.
 *  - Host-checkable errors (shape, dtype, stride, NULL, unsupported option)
 *    return before any launch with a message in dsv4_last_error().  Device
 *    contents (index ranges, page ids, qo_indptr[B] == T, n_q <= seq_len) are
 *    a caller contract; with DSV4_VALIDATE=1 in the environment the library
 *    copies them to the host (synchronously) and checks them first.
 *  - Split partial results go to one library workspace per device.  Calls on
 *    one device whose kernels could run at the same time (different streams
 *    without an ordering between them) race on it and give wrong results:
 *    serialise them (one stream, or events between streams).
 */
#ifndef DSV4_ATTN_H_
#define DSV4_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSV4_ABI_VERSION 2

/* Element types of a descriptor. */
enum {
    DSV4_BF16 = 1, /* bfloat16, 2 bytes */
    DSV4_F32 = 2,  /* float32 */
    DSV4_I32 = 3,  /* int32 */
    DSV4_U8 = 4    /* raw bytes (packed FP8 KV pages) */
};

typedef enum {
    DSV4_OK = 0,
    DSV4_ERR_INVALID = 1,     /* bad shape, dtype, stride, NULL, range */
    DSV4_ERR_UNSUPPORTED = 2, /* compress_ratio not in {0,4,128}, mixed pool formats, ... */
    DSV4_ERR_WORKSPACE = 3,   /* workspace allocation failed */
    DSV4_ERR_HIP = 4,         /* a HIP runtime call or launch failed */
    DSV4_ERR_CONTRACT = 5     /* DSV4_VALIDATE=1 found a device-content violation */
} dsv4_status;

typedef struct dsv4_tensor {
    void* data;
    int32_t dtype;     /* DSV4_* */
    int32_t ndim;      /* 1..4 */
    int64_t shape[4];
    int64_t stride[4]; /* in elements */
} dsv4_tensor;

/*
 * KV pool formats (both pools of one call must use the same one):
 *  - bf16:  DSV4_BF16 [S, 512], S = pages * 256, row stride a multiple of 8.
 *  - fp8:   DSV4_U8 [pages, 149504] contiguous.  Each 256-token page holds 256
 *           records of 576 bytes [448 x OCP E4M3FN non-rotary | 64 x bf16
 *           rotary], then 256 fp32 per-token scales (non-rotary value = code x
 *           scale), then 1 KiB of padding: 584 bytes per token (test-matrix
 *           page, "packed FP8 nope + BF16 rope", 584 bytes/token).
 */
#define DSV4_HEAD_DIM 512
#define DSV4_PAGE_SIZE 256
#define DSV4_FP8_PAGE_BYTES 149504

/*
 * dsv4_attn_forward -- SWA + (C4 | C128) attention for all query rows in one
 * call (overview page, kernel section: one call covers SWA and the extra
 * attention with shared metadata).
 *
 *  q                bf16 [T, H, 512], 1 <= H <= 128, inner strides multiples of 8
 *  swa_pool         KV pool (format above) holding the SWA cache
 *  swa_page_table   i32 [B, P_swa]: logical page x/256 -> physical page
 *  extra_pool       KV pool of compressed entries; ignored (may be NULL) if R == 0
 *  extra_page_table i32 [B, P_extra]; ignored (may be NULL) if R == 0
 *  c4_indices       i32 [T, K] logical compressed positions, -1 = unused;
 *                   required iff R == 4, ignored otherwise
 *  seq_lens         i32 [B]: total length including this pass's rows
 *  qo_indptr        i32 [B+1]: qo_indptr[0] = 0, non-decreasing, [B] = T
 *  sink             f32 [H] logits, or NULL (no sink)
 *  compress_ratio   0, 4 or 128 (else DSV4_ERR_UNSUPPORTED)
 *  window           W >= 1 (128 in DeepSeek-V4)
 *  scale            multiplies q.k (e.g. 512^-0.5); not applied to sink
 *  out              bf16 [T, H, 512], written (round to nearest even)
 *  lse              f32 [T, H] natural-log normaliser including the sink, or NULL
 *  stream           hipStream_t
 */
dsv4_status dsv4_attn_forward(const dsv4_tensor* q, const dsv4_tensor* swa_pool, const dsv4_tensor* swa_page_table,
                              const dsv4_tensor* extra_pool, const dsv4_tensor* extra_page_table,
                              const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens,
                              const dsv4_tensor* qo_indptr, const dsv4_tensor* sink, int32_t compress_ratio,
                              int32_t window, float scale, const dsv4_tensor* out, const dsv4_tensor* lse,
                              void* stream);

/*
 * dsv4_attn_forward_noalloc -- dsv4_attn_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, kernels, plan and
 * results as dsv4_attn_forward, but it never allocates: the split partials go
 * to a static per-device scratch array of dsv4_attn_noalloc_scratch_bytes()
 * bytes (32 MiB) that the library's code object holds on every device it is
 * loaded on until the process ends.  A call whose partials would not fit
 * (T x splits x H x 1028 bytes; splits from dsv4_attn_plan) returns
 * DSV4_ERR_WORKSPACE before any launch.  Every call on a device shares that
 * device's scratch: calls on one device that could run at the same time
 * (different streams without an ordering between them) race and give wrong
 * results.  The timing hook does not apply to this entry point.
 */
dsv4_status dsv4_attn_forward_noalloc(const dsv4_tensor* q, const dsv4_tensor* swa_pool,
                                      const dsv4_tensor* swa_page_table, const dsv4_tensor* extra_pool,
                                      const dsv4_tensor* extra_page_table, const dsv4_tensor* c4_indices,
                                      const dsv4_tensor* seq_lens, const dsv4_tensor* qo_indptr,
                                      const dsv4_tensor* sink, int32_t compress_ratio, int32_t window, float scale,
                                      const dsv4_tensor* out, const dsv4_tensor* lse, void* stream);

/* Size in bytes of the no-allocation entry point's static scratch. */
size_t dsv4_attn_noalloc_scratch_bytes(void);

/*
 * dsv4_kv_pack_fp8 -- the KV store in front of the attention: n new K rows
 * (with RoPE applied; V = K) quantised into packed FP8 records at given slots
 * (the cache write of the walk-through page, section 3; the 584-byte FP8 +
 * bf16 record of the test-matrix page, "packed FP8 nope + BF16 rope").
 *
 *  k      bf16 [n, 512], rows 16-byte aligned (row stride a multiple of 8)
 *  slots  i32 [n]: physical slot of row i (page slot/256, record slot%256), or
 *         < 0 to skip the row; the non-negative slots must be distinct and
 *         below pages*256 (a caller contract, checked with DSV4_VALIDATE=1)
 *  pool   DSV4_U8 [pages, 149504] packed FP8 pool (format above), written:
 *         for each row, scale = max |k[0..447]| / 448 in fp32 (1 if all
 *         those dims are zero); record bytes 0..447 = the OCP E4M3FN code of
 *         k[d] / scale (fp32 division), rounded to the nearest finite value,
 *         ties to the even code, saturating at +-448, sign from the sign bit;
 *         bytes 448..575 = k[448..511] unchanged; the page's fp32 scale of the
 *         record = scale.  Nothing else in the pool is touched.  k must be
 *         finite.
 *  stream hipStream_t
 *
 * A pool written here is read back exactly by dsv4_attn_forward (code x
 * scale).  Returns DSV4_ERR_UNSUPPORTED for a bf16 pool.
 */
dsv4_status dsv4_kv_pack_fp8(const dsv4_tensor* k, const dsv4_tensor* slots, const dsv4_tensor* pool, void* stream);

/*
 * dsv4_c4_topk -- the C4 index lists in front of the attention: per query
 * row, the K candidate compressed entries with the highest indexer scores
 * (overview page, "what V4 changed": the indexer keeps the top 512
 * compressed entries per query; its kernel section names a TopK kernel).
 *
 *  scores          f32 [T, ld]: scores[t][c] of candidate c (finite); only
 *                  c < num_candidates[t] is used (scores up to ld may be
 *                  read, never used)
 *  num_candidates  i32 [T]: candidates of row t, 0 <= n <= ld (for C4 at
 *                  position p, floor((p+1)/4)); a caller contract, checked
 *                  with DSV4_VALIDATE=1
 *  indices         i32 [T, K], 1 <= K <= 2048, written: the kept candidates
 *                  in ascending order, then -1 (all n when n <= K).  Kept: the
 *                  K highest scores; of equal scores the lower index first;
 *                  -0.0 equals +0.0.  The result is the c4_indices argument
 *                  of dsv4_attn_forward.
 *  stream          hipStream_t
 *
 * Rows of ld >= 32768 candidates (up to 65535 rows) use several workgroups
 * per row: the scores are read once, each 16384-candidate chunk appends its
 * own top K to the row's list in the library workspace (about 8 x (K + 1024)
 * bytes per chunk; see dsv4_attn_workspace_reserve: it grows on demand,
 * never under stream capture, and calls that could run at the same time on
 * one device race on it), and one workgroup per row selects from the list.
 */
dsv4_status dsv4_c4_topk(const dsv4_tensor* scores, const dsv4_tensor* num_candidates, const dsv4_tensor* indices,
                         void* stream);

/*
 * dsv4_attn_gather_slots -- the paged gather stage on its own: for every row,
 * the physical slots the attention reads, in canonical order (SWA positions
 * ascending, then C4 entries in index-list order with -1 skipped, or C128
 * entries ascending).  Same metadata arguments and contract as
 * dsv4_attn_forward (reference: the per-q-token SWA / C4 / C128 page-index
 * metadata of the test-matrix page, "reference implementation notes").
 *
 *  num_rows  T (rows of c4_indices / of the pass)
 *  slots     i32 [T, Kmax], Kmax >= window + (R==4 ? K : R==128 ? 256*P_extra : 0);
 *            entries past the row's count are set to -1
 *  counts    i32 [T, 2]: (number of SWA slots, number of extra slots)
 */
dsv4_status dsv4_attn_gather_slots(const dsv4_tensor* swa_page_table, const dsv4_tensor* extra_page_table,
                                   const dsv4_tensor* c4_indices, const dsv4_tensor* seq_lens,
                                   const dsv4_tensor* qo_indptr, int32_t num_rows, int32_t compress_ratio,
                                   int32_t window, const dsv4_tensor* slots, const dsv4_tensor* counts,
                                   void* stream);

/* Message of the last non-OK return on this thread ("" if none). */
const char* dsv4_last_error(void);

/* ABI version of the loaded library (DSV4_ABI_VERSION). */
int32_t dsv4_abi_version(void);

/*
 * Library workspace for split-KV partial results, one per device (split
 * kernel -> merge kernel).  dsv4_attn_forward grows it on demand with
 * hipMalloc (which synchronises the device), except while `stream` is being
 * captured into a HIP graph: then it never allocates and returns
 * DSV4_ERR_WORKSPACE if the workspace is too small.  A buffer replaced by a
 * larger one is kept until dsv4_attn_workspace_release, so graphs captured
 * earlier stay valid.
 *
 * dsv4_attn_workspace_reserve makes the current device's workspace at least
 * `bytes` large (call it, outside any capture, with the largest size the
 * captured calls need: T x splits x H x 1028 bytes, splits from
 * dsv4_attn_plan) and sets up the rest of the library's per-device state, so
 * that a graph may capture the process's first forward call.  `stream` is the
 * stream the caller is about to capture (used to refuse growth under
 * capture).  dsv4_attn_workspace_release synchronises every device that holds
 * a workspace and frees it; graphs that captured forward calls must not be
 * replayed afterwards.
 */
dsv4_status dsv4_attn_workspace_reserve(size_t bytes, void* stream);
void dsv4_attn_workspace_release(void);

/*
 * Tuning / test hook: force the number of keys handled by one split
 * (a positive multiple of 16 up to 2048), or 0 for the automatic plan.  The
 * kernel that runs rounds it up to its own tile (32 keys for the 32- and
 * 64-head variants and FP8, 16 for the 16-head variant) and caps it at its
 * own limit (1024 keys; 2048 for the 16-head variant).  Process-wide.
 */
dsv4_status dsv4_attn_set_split_keys(int32_t keys_per_split);

/*
 * Split-kernel variants.  Every variant computes the same attention; they
 * differ in how a workgroup of four waves divides its heads and head dims:
 *   DSV4_KERNEL_H16        16 heads per workgroup, four independent waves on
 *                          alternate 16-key tiles;
 *   DSV4_KERNEL_H32        32 heads, each wave one quarter of the head dims;
 *   DSV4_KERNEL_H32_ROLES  32 heads, two waves compute the scores and the
 *                          softmax (one dim half each), two accumulate P.V
 *                          (one dim half each);
 *   DSV4_KERNEL_H64        64 heads, two head groups x two dim halves;
 *   DSV4_KERNEL_FP8        packed FP8 pools: 64 heads, two head groups x two
 *                          dim halves;
 *   DSV4_KERNEL_FP8_H32    packed FP8 pools: 32 heads, each wave one quarter
 *                          of the head dims.
 * bf16 pools run one of the first four, packed FP8 pools one of the last two.
 */
enum {
    DSV4_KERNEL_AUTO = 0,
    DSV4_KERNEL_H16 = 1,
    DSV4_KERNEL_H32 = 2,
    DSV4_KERNEL_H32_ROLES = 3,
    DSV4_KERNEL_H64 = 4,
    DSV4_KERNEL_FP8 = 5,
    DSV4_KERNEL_FP8_H32 = 6
};

/*
 * Tuning / test hook: force a split-kernel variant, or DSV4_KERNEL_AUTO for
 * the automatic choice.  A forced bf16 variant (DSV4_KERNEL_H16 ..
 * DSV4_KERNEL_H64) applies to calls on bf16 pools only, a forced FP8 variant
 * (DSV4_KERNEL_FP8, DSV4_KERNEL_FP8_H32) to calls on packed FP8 pools only;
 * calls on the other format keep their automatic choice.  Any other value
 * returns DSV4_ERR_INVALID.  Process-wide.
 */
dsv4_status dsv4_attn_set_kernel(int32_t kernel);

/*
 * Plan that dsv4_attn_forward would use for these sizes: number of key
 * splits per (row, head block), keys per split, and the split-kernel variant
 * (DSV4_KERNEL_*; its heads per workgroup are 16, 32, 32, 64, 64 or 32).  kv_fp8
 * is nonzero for packed FP8 pools (the two formats run different kernels and
 * are planned differently).  kernel may be NULL.  Host-only, no device
 * access.
 */
dsv4_status dsv4_attn_plan(int32_t num_rows, int32_t num_heads, int32_t compress_ratio, int32_t window,
                           int32_t c4_width, int32_t extra_pages, int32_t kv_fp8, int32_t* splits,
                           int32_t* keys_per_split, int32_t* kernel);

/*
 * Kernel timing on the caller's stream with HIP events.  While enabled, every
 * dsv4_attn_forward records an event before the split kernel, one between it
 * and the merge kernel, and one after the merge kernel (only when a row is
 * split: otherwise there is no merge kernel and its time counts as 0).  The
 * events are timing-only (created without the system-scope fence on record),
 * so they neither flush caches nor stall the work that follows.  Calls made
 * while the stream is being captured into a HIP graph record external event
 * nodes instead, re-recorded on every replay.  dsv4_attn_timing_read waits
 * for the recorded events and returns the summed milliseconds of the split
 * kernels and of the merge kernels (either pointer may be NULL) and the
 * number of calls recorded, then clears the record; for graph-captured calls
 * it reports the most recent replay.  An interval holds its kernel plus the
 * events' own cost (a few percent of a 20 us kernel).
 */
dsv4_status dsv4_attn_timing_enable(int32_t enable);
dsv4_status dsv4_attn_timing_read(double* split_ms, double* merge_ms, int64_t* calls);

/*
 * Timing helper, not part of the attention: a plain streaming read of
 * `bytes` bytes of device memory at `buf`, launched on `stream`, for
 * measuring how fast this device reads a given number of bytes with nothing
 * else to do (no metadata to resolve, no arithmetic, no stores) -- the
 * yardstick beside the attention kernels' own rates.  `workgroups`
 * workgroups of 256 threads each read one contiguous share with 16-byte
 * non-temporal loads.  `sink` (device memory, 16 bytes) receives a store
 * only if the folded bytes equal one fixed 128-bit constant (it exists so
 * that the loads are kept); the caller owns both buffers.  Errors:
 * DSV4_ERR_INVALID for bytes negative or not a multiple of 16, workgroups
 * outside 1 .. 2^20, or a null or unaligned buf / sink (bytes = 0 launches
 * nothing); DSV4_ERR_HIP if the launch fails.
 */
dsv4_status dsv4_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink, void* stream);

/*
 * Test hook, not for production calls: record the KV rows the split kernels
 * read.  While `keys` is non-NULL, dsv4_attn_forward launches the recording
 * build of its split kernel (the same source, plus stores of what it
 * resolved), which writes for each work item -- row t, head block b of
 * dsv4_attn_plan's kernel, split s -- and each key k of the split
 * (0 <= k < keys_per_split, in the kernel's own key order):
 *   keys[((t * head_blocks + b) * splits + s) * keys_per_split + k]
 *       (uint64) = device address of the KV row it copied for that key
 *       (for packed FP8, the row's 576-byte record); the library's zero row
 *       for an unused C4 entry or a key past the split's end;
 *   masks[((t * head_blocks + b) * splits + s) * 32 + tile]
 *       (uint32, DSV4_KERNEL_H32 / _H32_ROLES / _H64 only) = the valid-key
 *       mask of each 32-key tile (bit k: key 32 * tile + k enters the softmax).
 * Entries a kernel does not reach keep their previous contents.  The
 * 32- and 64-head kernels walk a split's compressed entries first, then its
 * window keys; the 16-head and FP8 kernels the window first.  keys_cap and
 * masks_cap are the buffers' entry counts; a forward call that would write
 * past them returns DSV4_ERR_INVALID.  NULL keys switches recording off.
 * Process-wide; device pointers.
 */
dsv4_status dsv4_attn_debug_keys(void* keys, int64_t keys_cap, void* masks, int64_t masks_cap);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_ATTN_H_ */
