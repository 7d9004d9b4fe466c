/*
 * pa_oracle.c -- CPU oracle for paged split-KV decode.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct statement of what the decode path computes.
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links or calls it, and it shares no source with the GPU kernels.
 *
 * Arithmetic: integers (64-bit intermediates) for the planner, IEEE double for attention, keys and
 * head dimensions summed in index order.  Multithreading only partitions independent
 * (request, kv-head) tasks, so results do not depend on the thread count.
 *
 * Sources (web pages, cited by title and section):
 *   [ATOM-2366] ROCm/ATOM PR #2366 "[MiniMax-M3] Route the paged decode to aiter's FlyDSL kernel
 *               with work planner": section 1 Motivation, section 3 Design, section 5 Test Result,
 *               review item 2 (work entry contents) and item 3 (plan capacity formula).
 *   [ATOM-2514] ROCm/ATOM PR #2514 "Fix(attention): adapt the FlyDSL paged decode to aiter #5809
 *               (explicit work plans)": Motivation and Design (2 x CU budget on every call).
 *   [RDNA-29]   opengfx1030/vllm-rdna PR #29 (mixed and MTP-verify batches): Change, item 1
 *               "Kernel: per-token causal decode" (the sliding window applies per token), and the
 *               Test Plan's window cases.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_INVALID 1

/* storage type codes used by the Python wrapper of this oracle */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8E4M3 2

/* ------------------------------------------------------------------------------------------ */
/* Element decoding                                                                            */
/* ------------------------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double orc_bf16_to_double(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 "fn" variant: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, largest finite magnitude 448.  Decoded from the bit
 * fields by the definition, not by any conversion routine. */
static double orc_fp8e4m3_to_double(uint8_t code) {
    int sign = (code >> 7) & 1;
    int exp = (code >> 3) & 0xF;
    int man = code & 0x7;
    double mag;
    if (exp == 0xF && man == 0x7) return NAN;
    if (exp == 0)
        mag = ldexp((double)man / 8.0, 1 - 7);           /* subnormal: 0.man x 2^(1-bias) */
    else
        mag = ldexp(1.0 + (double)man / 8.0, exp - 7);   /* normal: 1.man x 2^(exp-bias) */
    return sign ? -mag : mag;
}

/* The 256 e4m3fn values, filled once from orc_fp8e4m3_to_double (a lookup, not a different rule). */
static double orc_fp8_table[256];
static pthread_once_t orc_fp8_once = PTHREAD_ONCE_INIT;
static void orc_fp8_fill(void) {
    for (int c = 0; c < 256; ++c) orc_fp8_table[c] = orc_fp8e4m3_to_double((uint8_t)c);
}

static double orc_load(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
        case ORC_F32: return (double)((const float*)base)[idx];
        case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
        case ORC_FP8E4M3: return orc_fp8_table[((const uint8_t*)base)[idx]];
        default: return NAN;
    }
}

int orc_decode_array(const void* src, int dtype, int64_t n, double* dst) {
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_FP8E4M3) return ORC_INVALID;
    pthread_once(&orc_fp8_once, orc_fp8_fill);
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_load(src, dtype, i);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O1: the length-proportional work planner                                                   */
/* ------------------------------------------------------------------------------------------ */

static int64_t orc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Plan capacity, as stated in [ATOM-2366] review item 3 and section 5 ("Planner drift at the real
 * ceiling"): min(batch x max_partitions, max(batch, ceil(budget x CU / kv_heads))), with the
 * budget of 2 x CU from [ATOM-2366] section 1 and [ATOM-2514] Design ("Default budget"). */
int orc_plan_capacity(int num_seqs, int num_kv_heads, int cu_count, int budget_mult,
                      int max_partitions, int32_t* capacity_out) {
    if (num_seqs < 0 || num_kv_heads < 1 || cu_count < 1 || budget_mult < 1 || max_partitions < 1)
        return ORC_INVALID;
    int64_t budget = orc_ceil_div((int64_t)budget_mult * cu_count, num_kv_heads);
    int64_t a = (int64_t)num_seqs * max_partitions;
    int64_t b = num_seqs > budget ? num_seqs : budget;
    int64_t c = a < b ? a : b;
    if (c > INT32_MAX) return ORC_INVALID;
    *capacity_out = (int32_t)c;
    return ORC_OK;
}

/* Key range a request reads: [lo_b, S_b).  Without a window, lo_b = 0.  With a window of W keys
 * (each token sees the last W of its visible keys, [RDNA-29] Change 1: the window applies per
 * token), the union over the request's L_b tokens starts at the first token's window:
 * lo_b = max(0, S_b - (L_b - 1) - W). */
static int64_t orc_read_start(int64_t S, int L, int window) {
    if (window <= 0) return 0;
    int64_t lo = S - (int64_t)(L - 1) - window;
    return lo > 0 ? lo : 0;
}

/* Work plan ([ATOM-2366] sections 1 and 3: each request receives a partition count proportional to
 * its real context length, under the workgroup budget, clamped only at max_partitions; work
 * entries carry begin/end tiles and the request's context length, [ATOM-2366] review item 2;
 * review "window logic": the plan must cover the key range the kernel reads under a window).
 *
 * Reading of the apportionment, which the pages leave open:
 *   the request reads keys [lo_b, S_b) (orc_read_start) and its tiles are the 256-token-aligned
 *   tiles that range touches: [floor(lo_b / T), ceil(S_b / T)), tiles_b of them;
 *   its length is E_b = S_b - lo_b (= S_b without a window); requests with E_b = 0 get no partition;
 *   every non-empty request gets one partition, and the capacity left over (C - B') is shared in
 *   proportion to E_b, rounded down:  parts_b = min(P, tiles_b, 1 + floor((C - B') E_b / W)),
 *   W = sum E_b;  any remainder is left unused.
 * Slots are filled request by request; partition j of request b spans tiles
 * [t0_b + floor(j tiles_b / parts_b), t0_b + floor((j+1) tiles_b / parts_b)), t0_b = floor(lo_b / T).
 * Unused slots hold (-1, 0, 0, 0).
 * work_info[slot] = (request, tile_begin, tile_end, S_b); reduce_info[b] = (first_slot, parts_b);
 * num_work = (used slots, tiles of the largest slot).
 * cu (nullable) gives the query lengths L_b; it only matters with a window.
 */
int orc_plan(const int32_t* context_lens, const int32_t* cu, int num_seqs, int num_kv_heads,
             int cu_count, int budget_mult, int max_partitions, int tile_tokens, int window,
             int capacity, int32_t* work_info, int32_t* reduce_info, int32_t* num_work) {
    int32_t cap = 0;
    if (tile_tokens < 1 || window < 0) return ORC_INVALID;
    if (orc_plan_capacity(num_seqs, num_kv_heads, cu_count, budget_mult, max_partitions, &cap))
        return ORC_INVALID;
    if (capacity < cap) return ORC_INVALID;
    for (int b = 0; b < num_seqs; ++b)
        if (context_lens[b] < 0) return ORC_INVALID;

    int64_t total = 0;        /* W */
    int64_t nonempty = 0;     /* B' */
    for (int b = 0; b < num_seqs; ++b) {
        int L = cu ? cu[b + 1] - cu[b] : 1;
        int64_t len = context_lens[b] - orc_read_start(context_lens[b], L, window);
        total += len;
        if (len > 0) nonempty += 1;
    }
    int64_t extra = (int64_t)cap - nonempty;

    int64_t slot = 0;
    int32_t largest = 0;
    for (int b = 0; b < num_seqs; ++b) {
        int64_t s = context_lens[b];
        int L = cu ? cu[b + 1] - cu[b] : 1;
        int64_t lo = orc_read_start(s, L, window);
        int64_t len = s - lo;
        int64_t t0 = lo / tile_tokens;
        int64_t parts = 0;
        int64_t tiles = len > 0 ? orc_ceil_div(s, tile_tokens) - t0 : 0;
        if (len > 0) {
            parts = 1 + (extra * len) / total;
            if (parts > tiles) parts = tiles;
            if (parts > max_partitions) parts = max_partitions;
        }
        if (slot + parts > capacity) return ORC_INVALID; /* never writes past the caller's buffer */
        reduce_info[2 * b + 0] = (int32_t)slot;
        reduce_info[2 * b + 1] = (int32_t)parts;
        for (int64_t j = 0; j < parts; ++j) {
            int32_t* w = work_info + 4 * (slot + j);
            w[0] = b;
            w[1] = (int32_t)(t0 + (j * tiles) / parts);
            w[2] = (int32_t)(t0 + ((j + 1) * tiles) / parts);
            w[3] = (int32_t)s;
            if (w[2] - w[1] > largest) largest = w[2] - w[1];
        }
        slot += parts;
    }
    if (slot > cap) return ORC_INVALID; /* cannot happen: sum of parts <= B' + extra = C */
    for (int64_t w = slot; w < capacity; ++w) {
        work_info[4 * w + 0] = -1;
        work_info[4 * w + 1] = 0;
        work_info[4 * w + 2] = 0;
        work_info[4 * w + 3] = 0;
    }
    num_work[0] = (int32_t)slot;
    num_work[1] = largest;
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O2 / O3: attention over the gathered pages                                                 */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    const void* q; int q_dtype; int num_rows; int num_q_heads; int head_dim;
    const void* k; const void* v; int kv_dtype; int num_blocks; int num_kv_heads; int block_size;
    const int32_t* block_tables; int max_blocks;
    const int32_t* context_lens; int num_seqs;
    const int32_t* cu; /* nullable */
    double scale, k_scale, v_scale;
    int window;        /* 0: none; W > 0: each token sees its last W visible keys */
} orc_problem;

/* Element (block, kv head, slot, d) of a paged cache laid out [num_blocks, Hkv, bs, D]. */
static int64_t orc_cache_index(const orc_problem* p, int64_t block, int g, int slot, int d) {
    return ((block * p->num_kv_heads + g) * p->block_size + slot) * (int64_t)p->head_dim + d;
}

/* Key position `pos` of request b -> physical block through the block table. */
static int64_t orc_page_of(const orc_problem* p, int b, int64_t pos) {
    return p->block_tables[(int64_t)b * p->max_blocks + pos / p->block_size];
}

/* Query tokens of request b and their first row.  Without cumulative query lengths every
 * request owns exactly one row, row b ([RDNA-29] Change 1: without cu_query_lens each token
 * reads its own row as before). */
static void orc_rows_of(const orc_problem* p, int b, int* first_row, int* qlen) {
    if (p->cu) {
        *first_row = p->cu[b];
        *qlen = p->cu[b + 1] - p->cu[b];
    } else {
        *first_row = b;
        *qlen = 1;
    }
}

/* Keys visible to token i of a request with L query tokens and KV length S: the first
 * S - (L - 1 - i), the causal range of [RDNA-29] Change 1. */
static int64_t orc_visible(int64_t S, int L, int i) { return S - (int64_t)(L - 1 - i); }

/* Start of token i's range: with a window of W keys the token sees [n - W, n) of its n visible
 * keys ([RDNA-29] Change 1: the sliding window applies per token); without one, [0, n). */
static int64_t orc_window_start(const orc_problem* p, int64_t n) {
    if (p->window <= 0) return 0;
    return n - p->window > 0 ? n - p->window : 0;
}

/* softmax-weighted sum over key positions [lo, hi) for one (row, head):
 * returns the partial (m, l, acc[D]) with m = max score, l = sum exp(s - m), acc = sum exp(s-m) v.
 * An empty range gives (-inf, 0, 0). */
static void orc_partial(const orc_problem* p, int b, int row, int h, int64_t lo, int64_t hi,
                        double* qv, double* scores, double* m_out, double* l_out, double* acc) {
    const int D = p->head_dim;
    const int G = p->num_q_heads / p->num_kv_heads;
    const int g = h / G; /* consecutive query heads share one kv head */
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    if (hi <= lo) { *m_out = -INFINITY; *l_out = 0.0; return; }
    for (int d = 0; d < D; ++d)
        qv[d] = orc_load(p->q, p->q_dtype, ((int64_t)row * p->num_q_heads + h) * D + d);
    double m = -INFINITY;
    for (int64_t pos = lo; pos < hi; ++pos) {
        int64_t blk = orc_page_of(p, b, pos);
        int slot = (int)(pos % p->block_size);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qv[d] * (orc_load(p->k, p->kv_dtype, orc_cache_index(p, blk, g, slot, d)) * p->k_scale);
        double s = p->scale * dot;
        scores[pos - lo] = s;
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t pos = lo; pos < hi; ++pos) {
        int64_t blk = orc_page_of(p, b, pos);
        int slot = (int)(pos % p->block_size);
        double w = exp(scores[pos - lo] - m);
        l += w;
        for (int d = 0; d < D; ++d)
            acc[d] += w * (orc_load(p->v, p->kv_dtype, orc_cache_index(p, blk, g, slot, d)) * p->v_scale);
    }
    *m_out = m;
    *l_out = l;
}

/* ---- thread fan-out over (request, kv head) tasks ---- */

typedef struct {
    const orc_problem* p;
    int mode;                 /* 0 = direct, 1 = split */
    const int32_t* work; const int32_t* reduce; int tile_tokens;
    double* out;
    int64_t max_ctx;
    int ntasks;
    int next;
    pthread_mutex_t mu;
    int status;
} orc_job;

static void orc_task_direct(orc_job* J, int b, int g, double* qv, double* scores, double* acc) {
    const orc_problem* p = J->p;
    const int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
    int row0, L;
    orc_rows_of(p, b, &row0, &L);
    int64_t S = p->context_lens[b];
    for (int i = 0; i < L; ++i) {
        int64_t n = orc_visible(S, L, i);
        for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            double* o = J->out + ((int64_t)(row0 + i) * p->num_q_heads + h) * D;
            if (n <= 0) { for (int d = 0; d < D; ++d) o[d] = 0.0; continue; }
            double m, l;
            orc_partial(p, b, row0 + i, h, orc_window_start(p, n), n, qv, scores, &m, &l, acc);
            for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
        }
    }
}

/* O3: partials per plan slot, then the log-sum-exp merge of a request's partials:
 * M = max_j m_j over partials with l_j > 0; out = sum_j e^{m_j-M} acc_j / sum_j e^{m_j-M} l_j. */
static void orc_task_split(orc_job* J, int b, int g, double* qv, double* scores, double* unused) {
    (void)unused;
    const orc_problem* p = J->p;
    const int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
    int row0, L;
    orc_rows_of(p, b, &row0, &L);
    int64_t S = p->context_lens[b];
    int first = J->reduce[2 * b], parts = J->reduce[2 * b + 1];
    double* pm = (double*)malloc(sizeof(double) * (parts > 0 ? parts : 1));
    double* pl = (double*)malloc(sizeof(double) * (parts > 0 ? parts : 1));
    double* pacc = (double*)malloc(sizeof(double) * (size_t)(parts > 0 ? parts : 1) * D);
    for (int i = 0; i < L; ++i) {
        int64_t n = orc_visible(S, L, i);
        for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            double* o = J->out + ((int64_t)(row0 + i) * p->num_q_heads + h) * D;
            for (int j = 0; j < parts; ++j) {
                const int32_t* w = J->work + 4 * (int64_t)(first + j);
                int64_t lo = (int64_t)w[1] * J->tile_tokens;
                int64_t hi = (int64_t)w[2] * J->tile_tokens;
                if (hi > w[3]) hi = w[3];
                if (hi > n) hi = n;
                if (lo < orc_window_start(p, n)) lo = orc_window_start(p, n);
                orc_partial(p, b, row0 + i, h, lo, hi, qv, scores, &pm[j], &pl[j], pacc + (int64_t)j * D);
            }
            double M = -INFINITY;
            for (int j = 0; j < parts; ++j)
                if (pl[j] > 0.0 && pm[j] > M) M = pm[j];
            double den = 0.0;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (n <= 0 || M == -INFINITY) continue; /* zero-length, empty range: the row is zero */
            for (int j = 0; j < parts; ++j) {
                if (!(pl[j] > 0.0)) continue;
                double f = exp(pm[j] - M);
                den += f * pl[j];
                for (int d = 0; d < D; ++d) o[d] += f * pacc[(int64_t)j * D + d];
            }
            for (int d = 0; d < D; ++d) o[d] /= den;
        }
    }
    free(pm); free(pl); free(pacc);
}

static void* orc_worker(void* arg) {
    orc_job* J = (orc_job*)arg;
    const orc_problem* p = J->p;
    double* qv = (double*)malloc(sizeof(double) * p->head_dim);
    double* acc = (double*)malloc(sizeof(double) * p->head_dim);
    double* scores = (double*)malloc(sizeof(double) * (size_t)(J->max_ctx > 0 ? J->max_ctx : 1));
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int t = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (t >= J->ntasks) break;
        int b = t / p->num_kv_heads, g = t % p->num_kv_heads;
        if (J->mode == 0) orc_task_direct(J, b, g, qv, scores, acc);
        else orc_task_split(J, b, g, qv, scores, acc);
    }
    free(qv); free(acc); free(scores);
    return NULL;
}

static int orc_check(const orc_problem* p) {
    if (p->window < 0) return ORC_INVALID;
    if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads) return ORC_INVALID;
    if (p->head_dim < 1 || p->block_size < 1 || p->num_seqs < 0 || p->num_rows < 0) return ORC_INVALID;
    int rows_used = p->cu ? p->cu[p->num_seqs] : p->num_seqs;
    if (rows_used > p->num_rows) return ORC_INVALID;
    for (int b = 0; b < p->num_seqs; ++b) {
        int64_t s = p->context_lens[b];
        if (s < 0 || orc_ceil_div(s, p->block_size) > p->max_blocks) return ORC_INVALID;
        if (p->cu && p->cu[b + 1] < p->cu[b]) return ORC_INVALID;
        for (int64_t pg = 0; pg < orc_ceil_div(s, p->block_size); ++pg) {
            int32_t blk = p->block_tables[(int64_t)b * p->max_blocks + pg];
            if (blk < 0 || blk >= p->num_blocks) return ORC_INVALID;
        }
    }
    return ORC_OK;
}

static int orc_run(orc_problem* p, int mode, const int32_t* work, const int32_t* reduce,
                   int tile_tokens, double* out, int nthreads) {
    if (orc_check(p)) return ORC_INVALID;
    pthread_once(&orc_fp8_once, orc_fp8_fill);
    const int64_t D = p->head_dim;
    /* rows not owned by any request (graph padding past the last cumulative length) are zero */
    memset(out, 0, sizeof(double) * (size_t)p->num_rows * p->num_q_heads * D);
    orc_job J;
    memset(&J, 0, sizeof J);
    J.p = p; J.mode = mode; J.work = work; J.reduce = reduce; J.tile_tokens = tile_tokens;
    J.out = out; J.ntasks = p->num_seqs * p->num_kv_heads;
    for (int b = 0; b < p->num_seqs; ++b)
        if (p->context_lens[b] > J.max_ctx) J.max_ctx = p->context_lens[b];
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, orc_worker, &J);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.mu);
    return ORC_OK;
}

#define ORC_PROBLEM_ARGS                                                                          \
    const void *q, int q_dtype, int num_rows, int num_q_heads, int head_dim, const void *k,      \
        const void *v, int kv_dtype, int num_blocks, int num_kv_heads, int block_size,           \
        const int32_t *block_tables, int max_blocks, const int32_t *context_lens, int num_seqs,  \
        const int32_t *cu, double scale, double k_scale, double v_scale, int window

#define ORC_FILL(p)                                                                               \
    orc_problem p = {q, q_dtype, num_rows, num_q_heads, head_dim, k, v, kv_dtype, num_blocks,     \
                     num_kv_heads, block_size, block_tables, max_blocks, context_lens, num_seqs,  \
                     cu, scale, k_scale, v_scale, window}

/* O2: direct softmax attention of every row over its visible keys, read through the block table. */
int orc_attention_direct(ORC_PROBLEM_ARGS, double* out, int nthreads) {
    ORC_FILL(p);
    return orc_run(&p, 0, NULL, NULL, 0, out, nthreads);
}

/* O3: attention computed per plan slot and merged; must equal O2 for any valid plan. */
int orc_attention_split(ORC_PROBLEM_ARGS, const int32_t* work_info, const int32_t* reduce_info,
                        int tile_tokens, double* out, int nthreads) {
    ORC_FILL(p);
    if (tile_tokens < 1) return ORC_INVALID;
    return orc_run(&p, 1, work_info, reduce_info, tile_tokens, out, nthreads);
}

/* O2 for a list of (row, head) pairs only, for spot checks of full-size outputs. */
int orc_attention_rows(ORC_PROBLEM_ARGS, const int32_t* rows, const int32_t* heads, int count,
                       double* out) {
    ORC_FILL(p);
    if (orc_check(&p)) return ORC_INVALID;
    pthread_once(&orc_fp8_once, orc_fp8_fill);
    const int D = head_dim;
    int64_t max_ctx = 1;
    for (int b = 0; b < num_seqs; ++b)
        if (context_lens[b] > max_ctx) max_ctx = context_lens[b];
    double* qv = (double*)malloc(sizeof(double) * D);
    double* scores = (double*)malloc(sizeof(double) * (size_t)max_ctx);
    int status = ORC_OK;
    for (int t = 0; t < count; ++t) {
        double* o = out + (int64_t)t * D;
        int r = rows[t], h = heads[t];
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (r < 0 || r >= num_rows || h < 0 || h >= num_q_heads) { status = ORC_INVALID; break; }
        /* which request owns row r: the last b with first_row(b) <= r < first_row(b) + L_b */
        int owner = -1, tok = 0, L = 1;
        for (int b = 0; b < num_seqs; ++b) {
            int r0, qlen;
            orc_rows_of(&p, b, &r0, &qlen);
            if (r >= r0 && r < r0 + qlen) { owner = b; tok = r - r0; L = qlen; break; }
        }
        if (owner < 0) continue; /* padding row */
        int64_t n = orc_visible(context_lens[owner], L, tok);
        if (n <= 0) continue;
        double m, l;
        orc_partial(&p, owner, r, h, orc_window_start(&p, n), n, qv, scores, &m, &l, o);
        for (int d = 0; d < D; ++d) o[d] /= l;
    }
    free(qv); free(scores);
    return status;
}
