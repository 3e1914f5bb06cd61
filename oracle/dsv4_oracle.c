/*
 * dsv4_oracle.c -- plain, slow fp64 CPU oracle for DeepSeek-V4 hybrid sparse
 * MQA attention (decode and target-verify).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so tests, the smoke check and the CPU baseline of
 * the benchmark can check the HIP library against an independent definition.
 * It shares no code, header, table or constant generator with the HIP path.
 *
 * What it computes (sources: the SGLang DSV4 attention test-matrix page and
 * the DSV4 attention walk-through page; the Day-0 overview page for the
 * per-layer architecture):
 *
 *  - Rows and positions (walk-through, sections 1 and 4 "Prefill and Decode
 *    metadata"): query row t belongs to the request r with
 *    qo_indptr[r] <= t < qo_indptr[r+1]; with n_q = qo_indptr[r+1]-qo_indptr[r]
 *    its position is p = seq_lens[r] - n_q + (t - qo_indptr[r]) (positions
 *    count from 0, length = last position + 1).
 *  - Keys (overview, "hybrid sparse attention"; walk-through section 5): every
 *    layer reads the sliding window of the last W tokens, x in [p-W+1, p], and
 *    according to compress_ratio R either nothing (R = 0), the C4 entries
 *    named by the row's top-k index list (R = 4), or every visible C128 entry
 *    (R = 128).  A compressed entry c is visible once its R source tokens are
 *    all at positions <= p, i.e. c < floor((p+1)/R).
 *  - Paging (test-matrix page, page_size 256 asserted): logical position x of
 *    request r lives at slot table[r][x / 256] * 256 + x % 256.
 *  - MQA with V = K (walk-through section 3: one shared KV head, the backend
 *    receives k = v): the value of a key is its full 512-wide row.
 *  - Attention sink (test-matrix page, "attention-sink correction"): one extra
 *    virtual key per head whose score is sink[h] and whose value is zero.
 *  - KV store (walk-through section 3, test-matrix page's packed FP8 record):
 *    dsv4o_pack_fp8 quantises K rows into packed FP8 records (see there).
 *
 *  out[t,h,:] = sum_k e^{s_k - m} K_k / (sum_k e^{s_k - m} + e^{sink_h - m}),
 *  s_k = scale * <q[t,h,:], K_k>,  lse = m + ln(denominator).
 *
 * Storage formats: bf16 rows are the upper 16 bits of an IEEE binary32; FP8
 * rows are OCP E4M3FN codes (bias 7, no infinities, S.1111.111 = NaN) times a
 * per-token fp32 scale for the 448 non-rotary dims, followed by 64 bf16
 * rotary dims.  Packed page layout: 256 records of 576 bytes, then 256 fp32
 * scales, then 1 KiB of padding (256 x 584 bytes).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).  Define DSV4O_MUTANT
 * to a positive number to compile a deliberately wrong variant; the tests use
 * those to show that the oracle's pins catch plausible mistakes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef DSV4O_MUTANT
#define DSV4O_MUTANT 0
#endif

#define O_PAGE 256
#define O_D 512
#define O_NOPE 448
#define O_ROPE 64
#define O_FP8_REC 576
#define O_FP8_SCALES (O_PAGE * O_FP8_REC)
#define O_FP8_PAGE (O_PAGE * 584)

typedef struct {
    int32_t B, T, H, W, R;
    int32_t kv_fp8;               /* 0: bf16 rows [pages*256, 512]; 1: packed fp8 pages */
    const int32_t* seq_lens;      /* [B] */
    const int32_t* qo_indptr;     /* [B+1] */
    const uint16_t* q;            /* [T, H, 512] bf16 bits */
    const float* sink;            /* [H] or NULL (no sink) */
    const uint8_t* swa_pool;
    int64_t swa_pool_pages;
    const int32_t* swa_page_table; /* [B, p_swa] */
    int32_t p_swa;
    const uint8_t* extra_pool;    /* NULL when R == 0 */
    int64_t extra_pool_pages;
    const int32_t* extra_page_table; /* [B, p_extra] */
    int32_t p_extra;
    const int32_t* c4_indices;    /* [T, K] when R == 4 */
    int32_t K;
    double scale;
} dsv4o_case;

static char g_err[512];
const char* dsv4o_last_error(void) { return g_err; }

static void set_err(const char* msg, long a, long b) {
#pragma omp critical(dsv4o_err)
    snprintf(g_err, sizeof g_err, "%s (%ld, %ld)", msg, a, b);
}

/* ---- storage decoding ---------------------------------------------------- */

double dsv4o_bf16_to_double(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN. */
double dsv4o_e4m3_to_double(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

static void decode_row(const dsv4o_case* c, const uint8_t* pool, int64_t slot, double* dst) {
    if (!c->kv_fp8) {
        const uint16_t* row = (const uint16_t*)pool + slot * O_D;
        for (int d = 0; d < O_D; ++d) dst[d] = dsv4o_bf16_to_double(row[d]);
        return;
    }
    int64_t page = slot / O_PAGE, rec = slot % O_PAGE;
    const uint8_t* base = pool + page * (int64_t)O_FP8_PAGE;
    const uint8_t* row = base + rec * O_FP8_REC;
    float sc;
    memcpy(&sc, base + O_FP8_SCALES + 4 * rec, sizeof sc);
#if DSV4O_MUTANT == 6
    sc = 1.0f; /* mutant: per-token scale not applied */
#endif
    for (int d = 0; d < O_NOPE; ++d) dst[d] = dsv4o_e4m3_to_double(row[d]) * (double)sc;
    for (int d = 0; d < O_ROPE; ++d) {
        uint16_t bits;
        memcpy(&bits, row + O_NOPE + 2 * d, sizeof bits);
        dst[O_NOPE + d] = dsv4o_bf16_to_double(bits);
    }
}

/* ---- rows, positions and key lists -------------------------------------- */

/* Request owning row t: the r with qo_indptr[r] <= t < qo_indptr[r+1]. */
static int row_request(const dsv4o_case* c, int32_t t) {
    for (int r = 0; r < c->B; ++r)
        if (c->qo_indptr[r] <= t && t < c->qo_indptr[r + 1]) return r;
    return -1;
}

static int row_position(const dsv4o_case* c, int32_t t, int* r_out, int64_t* p_out) {
    int r = row_request(c, t);
    if (r < 0) { set_err("row outside qo_indptr", t, c->T); return -1; }
    int64_t n_q = (int64_t)c->qo_indptr[r + 1] - c->qo_indptr[r];
    int64_t L = c->seq_lens[r];
    if (n_q > L) { set_err("more query rows than tokens in request", r, L); return -1; }
    int64_t p = L - n_q + (t - c->qo_indptr[r]);
#if DSV4O_MUTANT == 2
    p = p - 1; /* mutant: positions shifted by one */
#endif
    *r_out = r;
    *p_out = p;
    return 0;
}

static int lookup_slot(const int32_t* table, int32_t width, int64_t pool_pages, int r, int64_t x,
                       int64_t* slot) {
#if DSV4O_MUTANT == 8
    int64_t lp = x % O_PAGE, off = x / O_PAGE; /* mutant: page and offset swapped */
#else
    int64_t lp = x / O_PAGE, off = x % O_PAGE;
#endif
    if (lp < 0 || lp >= width) { set_err("logical page outside page table", r, (long)x); return -1; }
    int32_t pg = table[(int64_t)r * width + lp];
    if (pg < 0 || pg >= pool_pages) { set_err("page table entry outside pool", r, pg); return -1; }
    *slot = (int64_t)pg * O_PAGE + off;
    return 0;
}

/*
 * Ordered key list of row t: SWA slots for x = max(0,p-W+1) .. p ascending,
 * then extra slots (C4: index-list order, -1 skipped; C128: c = 0 .. vis-1).
 * Returns 0 and fills the counts, or -1 on a caller-contract violation.
 * The slot arrays must hold W and max(K, p_extra*256) entries.
 */
int dsv4o_gather(const dsv4o_case* c, int32_t t, int32_t* swa_slots, int32_t* n_swa, int32_t* extra_slots,
                 int32_t* n_extra) {
    int r;
    int64_t p;
    if (row_position(c, t, &r, &p)) return -1;
    int64_t lo = p - c->W + 1;
#if DSV4O_MUTANT == 1
    lo = p - c->W; /* mutant: window one token too wide */
#endif
    if (lo < 0) lo = 0;
    int ns = 0;
    for (int64_t x = lo; x <= p; ++x) {
        int64_t s;
        if (lookup_slot(c->swa_page_table, c->p_swa, c->swa_pool_pages, r, x, &s)) return -1;
        swa_slots[ns++] = (int32_t)s;
    }
    int ne = 0;
    if (c->R == 4) {
        int64_t vis = (p + 1) / 4;
        const int32_t* idx = c->c4_indices + (int64_t)t * c->K;
#if DSV4O_MUTANT == 9
        idx = c->c4_indices + (int64_t)c->qo_indptr[r] * c->K; /* mutant: first row's list for all rows */
#endif
        for (int k = 0; k < c->K; ++k) {
            int64_t e = idx[k];
            if (e < 0) continue;
            if (e >= vis) { set_err("C4 index not visible to row", t, (long)e); return -1; }
            int64_t s;
            if (lookup_slot(c->extra_page_table, c->p_extra, c->extra_pool_pages, r, e, &s)) return -1;
            extra_slots[ne++] = (int32_t)s;
        }
    } else if (c->R == 128) {
        int64_t vis = (p + 1) / 128;
#if DSV4O_MUTANT == 7
        vis = p / 128; /* mutant: last complete block hidden */
#endif
        for (int64_t e = 0; e < vis; ++e) {
            int64_t s;
            if (lookup_slot(c->extra_page_table, c->p_extra, c->extra_pool_pages, r, e, &s)) return -1;
            extra_slots[ne++] = (int32_t)s;
        }
    } else if (c->R != 0) {
        set_err("compress ratio must be 0, 4 or 128", c->R, 0);
        return -1;
    }
    *n_swa = ns;
    *n_extra = ne;
    return 0;
}

/* ---- attention ------------------------------------------------------------ */

static int attend_row(const dsv4o_case* c, int32_t t, double* out, double* lse, double* lse_nosink) {
    int32_t cap_e = c->K > c->p_extra * O_PAGE ? c->K : c->p_extra * O_PAGE;
    int32_t* swa = (int32_t*)malloc(sizeof(int32_t) * (size_t)(c->W > 0 ? c->W + 1 : 1));
    int32_t* ext = (int32_t*)malloc(sizeof(int32_t) * (size_t)(cap_e > 0 ? cap_e : 1));
    int32_t ns = 0, ne = 0;
    int rc = dsv4o_gather(c, t, swa, &ns, ext, &ne);
    if (rc) { free(swa); free(ext); return rc; }
    int n = ns + ne;
    double* keys = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * O_D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int k = 0; k < ns; ++k) decode_row(c, c->swa_pool, swa[k], keys + (size_t)k * O_D);
    for (int k = 0; k < ne; ++k) decode_row(c, c->extra_pool, ext[k], keys + (size_t)(ns + k) * O_D);

    for (int h = 0; h < c->H; ++h) {
        const uint16_t* qh = c->q + ((int64_t)t * c->H + h) * O_D;
        double qd[O_D];
        for (int d = 0; d < O_D; ++d) qd[d] = dsv4o_bf16_to_double(qh[d]);
#if DSV4O_MUTANT == 5
        for (int d = O_NOPE; d < O_D; ++d) qd[d] = 0.0; /* mutant: rotary dims left out of the score */
#endif
        double smax = -INFINITY;
        for (int k = 0; k < n; ++k) {
            const double* kr = keys + (size_t)k * O_D;
            double acc = 0.0;
            for (int d = 0; d < O_D; ++d) acc += qd[d] * kr[d];
#if DSV4O_MUTANT == 12
            s[k] = acc; /* mutant: softmax scale not applied */
#else
            s[k] = c->scale * acc;
#endif
            if (s[k] > smax) smax = s[k];
        }
        double sig = c->sink ? (double)c->sink[h] : -INFINITY;
#if DSV4O_MUTANT == 3
        sig = c->sink ? c->scale * (double)c->sink[h] : -INFINITY; /* mutant: sink scaled like a score */
#endif
        double m = smax > sig ? smax : sig;
        double zk = 0.0;
        for (int k = 0; k < n; ++k) zk += exp(s[k] - m);
        double zs = (sig == -INFINITY) ? 0.0 : exp(sig - m);
#if DSV4O_MUTANT == 4
        zs = 0.0; /* mutant: sink left out of the denominator */
#endif
        double z = zk + zs;
        double* oh = out + (size_t)h * O_D;
        for (int d = 0; d < O_D; ++d) oh[d] = 0.0;
        for (int k = 0; k < n; ++k) {
            double w = exp(s[k] - m) / z;
            const double* kr = keys + (size_t)k * O_D;
            for (int d = 0; d < O_D; ++d) oh[d] += w * kr[d];
        }
#if DSV4O_MUTANT == 11
        for (int d = O_NOPE; d < O_D; ++d) oh[d] = 0.0; /* mutant: value restricted to non-rotary dims */
#endif
        lse[h] = m + log(z);
        /* without the sink: max over real keys only */
        double zn = 0.0;
        for (int k = 0; k < n; ++k) zn += exp(s[k] - smax);
        lse_nosink[h] = smax + log(zn);
#if DSV4O_MUTANT == 10
        lse[h] = lse_nosink[h]; /* mutant: lse reported without the sink */
#endif
    }
    free(keys);
    free(s);
    free(swa);
    free(ext);
    return 0;
}

/*
 * Attention for the listed rows.  out: [nrows, H, 512], lse and lse_nosink:
 * [nrows, H], all fp64.  nthreads <= 0 uses the OpenMP default.  Returns 0,
 * or -1 with dsv4o_last_error() set when an input breaks the caller contract.
 */
int dsv4o_attention(const dsv4o_case* c, const int32_t* rows, int32_t nrows, double* out, double* lse,
                    double* lse_nosink, int32_t nthreads) {
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nrows; ++i) {
        int rc = attend_row(c, rows[i], out + (size_t)i * c->H * O_D, lse + (size_t)i * c->H,
                            lse_nosink + (size_t)i * c->H);
        if (rc) {
#pragma omp atomic write
            failed = 1;
        }
    }
    return failed ? -1 : 0;
}

/* ---- KV store: the packed FP8 record -------------------------------------- */

/* Nearest finite OCP E4M3FN value to x, by search over the 127 non-negative
 * finite codes; of two equally near values the one with the even code (even
 * mantissa) wins; beyond the largest finite value (448) the nearest one is
 * 448, so large magnitudes saturate.  The sign of the code is the sign bit
 * of x (-0.0 and negatives that round to zero give 0x80).  x must be finite. */
uint8_t dsv4o_e4m3_from_float(float x) {
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    const double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int code = 0; code < 0x7F; ++code) {
        const double d = fabs(dsv4o_e4m3_to_double((uint8_t)code) - a);
#if DSV4O_MUTANT == 13
        if (d < best_d || (d == best_d && code > best)) {  /* ties away from zero */
#else
        if (d < best_d || (d == best_d && (code & 1) == 0)) {
#endif
            best = code;
            best_d = d;
        }
    }
    return (uint8_t)(best | ((bits >> 31) << 7));
}

/* The cache write of the walk-through page (section 3, k = v) into the packed
 * FP8 record of the test-matrix page (448 E4M3FN non-rotary codes + 64 bf16
 * rotary dims + an fp32 per-token scale, 584 bytes/token; the record layout
 * inside a page is this library's, see dsv4_attn.h).  Row i of k (bf16 bits
 * [n, 512]) goes to slot slots[i] of the pool, or nowhere if slots[i] < 0:
 *   scale  = max_d |nope_d| / 448 in float (1 if every nope dim is zero),
 *   code_d = the E4M3FN code nearest to nope_d / scale (float division),
 *   rope   = the 64 rotary bf16 values unchanged.
 * The float divisions are the reading both the oracle and the kernel take,
 * so that every code is decided from the same value. */
int dsv4o_pack_fp8(const uint16_t* k, const int32_t* slots, int64_t n, uint8_t* pool, int64_t pool_pages) {
    for (int64_t i = 0; i < n; ++i) {
        const int32_t slot = slots[i];
        if (slot < 0) continue;
        const int64_t page = slot / O_PAGE, rec = slot % O_PAGE;
        if (page >= pool_pages) {
            set_err("pack: slot %ld beyond the pool's %ld pages", (long)slot, (long)pool_pages);
            return -1;
        }
        const uint16_t* row = k + i * O_D;
        float nope[O_NOPE];
        float amax = 0.f;
        for (int d = 0; d < O_NOPE; ++d) {
            nope[d] = (float)dsv4o_bf16_to_double(row[d]);
            amax = fmaxf(amax, fabsf(nope[d]));
        }
#if DSV4O_MUTANT == 14
        const float scale = amax > 0.f ? amax / 447.0f : 1.0f;  /* wrong divisor */
#else
        const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#endif
        uint8_t* dst = pool + page * O_FP8_PAGE + rec * O_FP8_REC;
        for (int d = 0; d < O_NOPE; ++d) dst[d] = dsv4o_e4m3_from_float(nope[d] / scale);
        for (int d = 0; d < O_ROPE; ++d) {
#if DSV4O_MUTANT == 15
            const uint16_t v = row[O_NOPE + (d ^ 1)];  /* rotary dims swapped in pairs */
#else
            const uint16_t v = row[O_NOPE + d];
#endif
            dst[O_NOPE + 2 * d] = (uint8_t)(v & 0xFF);
            dst[O_NOPE + 2 * d + 1] = (uint8_t)(v >> 8);
        }
        memcpy(pool + page * O_FP8_PAGE + O_FP8_SCALES + 4 * rec, &scale, 4);
    }
    return 0;
}

int dsv4o_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int dsv4o_mutant(void) { return DSV4O_MUTANT; }
