/*
 * CPU oracle for the FP4 lightning indexer with the hierarchical candidate pool.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code, header, table or constant with the GPU library.
 *
 * Plain, slow and direct: no blocking, no SIMD, no BLAS. Floating point is fp64 except where
 * the method fixes a narrower precision (the rotation output feeds the FP4 encoder as fp32).
 *
 * Sources (web pages on DeepSeek-V4.1's indexer, cited by title and section):
 *  [P1] "DeepSeek-V4.1 model structure (3): sequence dimension, Hierarchical Sparse Indexer and
 *       FP4 KV cache" (blog.javazero.top): the indexer score equation (section "Reindex layers
 *       score a million entries per token"), the candidate pool (section "use shallow scores to
 *       limit deep scoring" and the code walk-through "three details of the pool"), the E2M1
 *       value set, the quantise/dequantise equation and the scale table (sections "E2M1 has only
 *       15 values" and "the scale format decides precision").
 *  [P3] "DeepSeek-V4 model structure (2): Lightning Indexer and sparse selection" (xhh.club):
 *       ReLU instead of softmax, query-generated head weights, FP4 with a random Hadamard
 *       rotation (Q&A on quantisation).
 *
 * Readings where the pages are silent (listed with reasons in the design notes):
 *  - random Hadamard = per-channel signs, then the orthonormal Sylvester transform of size 128,
 *    the same signs for q and k; output rounded to fp32 as fl32(fl32(S) * fl32(2^-3.5)) where S
 *    is the exact signed sum;
 *  - UE8M0 scale exponent e = the smallest integer with 6 * 2^e >= max|y| of the 32-group
 *    ("rounded up to a power of two" in [P1]); an all-zero group gets e = -127;
 *  - E2M1 rounding: nearest representable magnitude, ties to the even mantissa bit; a value that
 *    rounds to zero is +0; element 2i is the low nibble of byte i;
 *  - top-k and pool ties go to the lower index; invisible positions never enter a selection.
 *
 *  - main KV ([P1] "the scale format decides precision" and "removing the global scale"): rows of
 *    512 values in groups of 16, one E4M3 (OCP "fn": no infinities, S.1111.111 is NaN) scale per
 *    group and no global scale; the scale is the smallest E4M3 value s with 6 * s >= max|x| of
 *    the group (the E8M0 rule's "rounded up", on the finer E4M3 grid), saturating at 448; an
 *    all-zero group gets s = 0 and zero codes; codes as for the indexer rows (nearest, ties to
 *    even, +0); 256 code bytes + 32 scale bytes per row;
 *
 * Parity pins (see tests/test_oracle_*.py): E2M1 value set and the rounding thresholds, scale
 * minimality, rotation against a library Hadamard matrix and orthogonality, per-head dot against
 * a dequantised fp64 dot, score special cases, brute-force selection on tiny inputs, the nesting
 * invariant, gather form = mask form, and the pages' MAC counts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define NHEAD 32
#define DIM 128
#define GROUP 32

/* ------------------------------------------------------------------ MAC counter */
static uint64_t g_macs = 0;
uint64_t orc_mac_count(void) { return __atomic_load_n(&g_macs, __ATOMIC_RELAXED); }
void orc_mac_reset(void) { __atomic_store_n(&g_macs, 0, __ATOMIC_RELAXED); }

/* ------------------------------------------------------------------ bf16 input */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------ rotation
 * y = H (sigma * x) / sqrt(128) with the Sylvester Hadamard matrix H[i][c] = (-1)^popcount(i&c).
 * The signed sum S_i is exact in fp64 (bf16 inputs, 128 terms); then two fp32 roundings.
 */
float orc_inv_sqrt128_f32(void) { return (float)(sqrt(2.0) / 16.0); }

void orc_rotate(const uint16_t* x, const int8_t* signs, float* y) {
    const float r = orc_inv_sqrt128_f32();
    for (int i = 0; i < DIM; ++i) {
        double s = 0.0;
        for (int c = 0; c < DIM; ++c) {
            double h = (__builtin_popcount((unsigned)(i & c)) & 1) ? -1.0 : 1.0;
            s += h * (double)signs[c] * bf16_value(x[c]);
        }
        float sf = (float)s;
        y[i] = sf * r; /* fp32 multiply, round to nearest even */
    }
}

/* ------------------------------------------------------------------ E2M1 / UE8M0 */
/* E2M1 magnitudes by code 0..7 ([P1] "E2M1 has only 15 values") */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* nearest representable magnitude (|v| <= 6 assumed by the scale rule), ties to the code with
 * an even mantissa bit; sign bit 3; a zero result is +0 */
int orc_e2m1_code(double v) {
    double a = fabs(v);
    int best = 0;
    double bd = fabs(a - E2M1_MAG[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - E2M1_MAG[c]);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    if (best != 0 && v < 0) best |= 8;
    return best;
}

/* smallest e with 6 * 2^e >= a, clamped to [-127, 127]; a == 0 gives -127 */
int orc_scale_exp(double a) {
    if (a == 0.0) return -127;
    int e = ilogb(a) - 3;
    while (ldexp(6.0, e) < a) ++e;
    while (ldexp(6.0, e - 1) >= a) --e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* quantise one rotated 128-row: codes[64] (element 2i low nibble of byte i), scales[4] = e+127 */
void orc_quantize_row(const float* y, uint8_t* codes, uint8_t* scales) {
    for (int g = 0; g < DIM / GROUP; ++g) {
        double a = 0.0;
        for (int c = 0; c < GROUP; ++c) {
            double v = fabs((double)y[g * GROUP + c]);
            if (v > a) a = v;
        }
        int e = orc_scale_exp(a);
        scales[g] = (uint8_t)(e + 127);
        for (int c = 0; c < GROUP; c += 2) {
            int lo = orc_e2m1_code(ldexp((double)y[g * GROUP + c], -e));
            int hi = orc_e2m1_code(ldexp((double)y[g * GROUP + c + 1], -e));
            codes[(g * GROUP + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

typedef struct {
    const uint16_t* x;
    const int8_t* signs;
    uint8_t* codes;
    uint8_t* scales;
    int64_t r0, r1;
} qjob;

static void* run_quant(void* p) {
    qjob* j = (qjob*)p;
    float y[DIM];
    for (int64_t r = j->r0; r < j->r1; ++r) {
        orc_rotate(j->x + r * DIM, j->signs, y);
        orc_quantize_row(y, j->codes + r * 64, j->scales + r * 4);
    }
    return NULL;
}

/* rotate + quantise rows of 128 bf16 values */
void orc_quantize_rows(const uint16_t* x, int64_t rows, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                       int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (rows < 256) nthreads = 1;
    pthread_t th[256];
    qjob jobs[256];
    int64_t per = (rows + nthreads - 1) / nthreads;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t a = per * t, b = a + per < rows ? a + per : rows;
        if (a >= b) break;
        jobs[t] = (qjob){x, signs, codes, scales, a, b};
        if (nthreads == 1) {
            run_quant(&jobs[t]);
        } else {
            pthread_create(&th[t], NULL, run_quant, &jobs[t]);
            ++used;
        }
    }
    for (int t = 0; t < used; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ per-head dot
 * Decode codes to signed half-units {0,1,2,3,4,6,8,12}; per group P_g = sum of products (integer,
 * quarter-units); d = sum_g P_g * 2^(eq_g + ek_g) / 4, summed exactly in int64 at the smallest
 * exponent of a nonzero group.
 *   returns 1 when d is exactly representable in fp32, else 0.
 *   *hw_spread = max_g (eq_g+ek_g) over all groups minus the smallest over nonzero groups.
 */
static const int HALF_UNITS[8] = {0, 1, 2, 3, 4, 6, 8, 12};

static inline int code_half(uint8_t byte, int hi) {
    int c = hi ? (byte >> 4) & 15 : byte & 15;
    int m = HALF_UNITS[c & 7];
    return (c & 8) ? -m : m;
}

int orc_head_dot(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, double* d,
                 int* hw_spread) {
    int64_t P[4];
    int E[4];
    for (int g = 0; g < 4; ++g) {
        int64_t s = 0;
        for (int c = 0; c < GROUP; ++c) {
            int idx = g * GROUP + c;
            s += (int64_t)code_half(qc[idx / 2], idx & 1) * (int64_t)code_half(kc[idx / 2], idx & 1);
        }
        P[g] = s;
        E[g] = ((int)qs[g] - 127) + ((int)ks[g] - 127);
    }
    __atomic_fetch_add(&g_macs, (uint64_t)DIM, __ATOMIC_RELAXED);
    int emin = 1 << 30, emax = -(1 << 30);
    for (int g = 0; g < 4; ++g) {
        if (E[g] > emax) emax = E[g];
        if (P[g] != 0 && E[g] < emin) emin = E[g];
    }
    if (emin == (1 << 30)) { /* every group product is zero */
        *d = 0.0;
        if (hw_spread) *hw_spread = 0;
        return 1;
    }
    if (hw_spread) *hw_spread = emax - emin;
    int nzmax = -(1 << 30);
    for (int g = 0; g < 4; ++g)
        if (P[g] != 0 && E[g] > nzmax) nzmax = E[g];
    if (nzmax - emin > 40) { /* cannot be summed exactly in int64; never happens on the workloads */
        double s = 0.0;
        for (int g = 0; g < 4; ++g) s += ldexp((double)P[g], E[g] - 2);
        *d = s;
        return 0;
    }
    int64_t tot = 0;
    for (int g = 0; g < 4; ++g)
        if (P[g] != 0) tot += P[g] * ((int64_t)1 << (E[g] - emin));
    *d = ldexp((double)tot, emin - 2); /* |tot| < 2^55 only if spread > 40, excluded above */
    if (tot == 0) {
        *d = 0.0;
        return 1;
    }
    /* fp32-representable: at most 24 significant bits and a normal-or-subnormal exponent */
    int64_t m = tot < 0 ? -tot : tot;
    while ((m & 1) == 0) m >>= 1;
    int bits = 0;
    while (m) {
        ++bits;
        m >>= 1;
    }
    return (bits <= 24 && (double)(float)*d == *d) ? 1 : 0;
}

/* ------------------------------------------------------------------ score
 * I = sum_j w_j * max(d_j, 0) (fp64, head order), A = sum_j |w_j| * max(d_j, 0).
 * q_codes: [32][64], q_scales: [32][4]; kc: [64]; ks: [4].
 */
double orc_score(const uint8_t* qc, const uint8_t* qs, const float* w, const uint8_t* kc, const uint8_t* ks,
                 double* A, double* dots) {
    double I = 0.0, a = 0.0;
    for (int j = 0; j < NHEAD; ++j) {
        double d;
        orc_head_dot(qc + j * 64, qs + j * 4, kc, ks, &d, NULL);
        if (dots) dots[j] = d;
        double r = d > 0.0 ? d : 0.0;
        I += (double)w[j] * r;
        a += fabs((double)w[j]) * r;
    }
    if (A) *A = a;
    return I + 0.0; /* canonical +0 */
}

/* scores of entries 0..n-1 of one query; dots (nullable) is [32][n] */
void orc_score_rows(const uint8_t* qc, const uint8_t* qs, const float* w, const uint8_t* kc, const uint8_t* ks,
                    int64_t n, double* I, double* A, double* dots) {
    double dj[NHEAD];
    for (int64_t s = 0; s < n; ++s) {
        double a;
        I[s] = orc_score(qc, qs, w, kc + s * 64, ks + s * 4, &a, dots ? dj : NULL);
        if (A) A[s] = a;
        if (dots)
            for (int j = 0; j < NHEAD; ++j) dots[(int64_t)j * n + s] = dj[j];
    }
}

/* ------------------------------------------------------------------ selection */
typedef struct {
    double v;
    int64_t i;
} vi_t;

static int cmp_desc(const void* pa, const void* pb) {
    const vi_t* a = (const vi_t*)pa;
    const vi_t* b = (const vi_t*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* top-k of the finite values I[0..n-1] by (value desc, index asc) via a full sort; out[k]
 * padded with -1; returns the number selected */
int32_t orc_topk(const double* I, int64_t n, int32_t k, int32_t* out) {
    vi_t* a = (vi_t*)malloc(sizeof(vi_t) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t s = 0; s < n; ++s)
        if (isfinite(I[s]) || I[s] == INFINITY) a[m++] = (vi_t){I[s], s};
    qsort(a, (size_t)m, sizeof(vi_t), cmp_desc);
    int32_t cnt = (int32_t)(m < k ? m : k);
    for (int32_t t = 0; t < k; ++t) out[t] = t < cnt ? (int32_t)a[t].i : -1;
    free(a);
    return cnt;
}

/* block maxima over blocks of `block` positions; positions >= n count as -inf; returns nb */
int64_t orc_block_max(const double* I, int64_t n, int32_t block, double* bm) {
    int64_t nb = (n + block - 1) / block;
    for (int64_t b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int64_t s = b * block; s < (b + 1) * block; ++s) {
            double v = s < n ? I[s] : -INFINITY;
            if (v > m) m = v;
        }
        bm[b] = m;
    }
    return nb;
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* candidate pool from raw block maxima: pin the block holding position n-1 to +inf, rank the
 * blocks by (value desc, block asc), keep the first min(topk_blocks, nb) whose value is above
 * -inf; out_blocks ascending; returns the count */
int32_t orc_pool(const double* bm, int64_t n, int32_t block, int32_t topk_blocks, int32_t* out_blocks) {
    int64_t nb = (n + block - 1) / block;
    if (nb <= 0) return 0;
    vi_t* a = (vi_t*)malloc(sizeof(vi_t) * (size_t)nb);
    int64_t last = (n - 1) / block;
    for (int64_t b = 0; b < nb; ++b) a[b] = (vi_t){b == last ? INFINITY : bm[b], b};
    qsort(a, (size_t)nb, sizeof(vi_t), cmp_desc);
    int64_t take = nb < topk_blocks ? nb : topk_blocks;
    int32_t cnt = 0;
    for (int64_t t = 0; t < take; ++t)
        if (a[t].v > -INFINITY) out_blocks[cnt++] = (int32_t)a[t].i;
    free(a);
    qsort(out_blocks, (size_t)cnt, sizeof(int32_t), cmp_i32);
    return cnt;
}

/* the pool as the official code applies it: every visible position outside the pooled blocks
 * set to -inf, pooled positions keep their score */
void orc_mask_pool(const double* I_full, int64_t n, const int32_t* pool_blocks, int32_t count, int32_t block,
                   double* m) {
    for (int64_t s = 0; s < n; ++s) m[s] = -INFINITY;
    for (int32_t i = 0; i < count; ++i)
        for (int64_t s = (int64_t)pool_blocks[i] * block; s < ((int64_t)pool_blocks[i] + 1) * block && s < n; ++s)
            if (s >= 0) m[s] = I_full[s];
}

/* Reindex, mask form: scores of every visible position, non-pool positions set to -inf, then
 * top-k of what is left */
int32_t orc_reindex_mask(const double* I_full, int64_t n, const int32_t* pool_blocks, int32_t count,
                         int32_t block, int32_t k, int32_t* out) {
    double* m = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    orc_mask_pool(I_full, n, pool_blocks, count, block, m);
    int32_t r = orc_topk(m, n, k, out);
    free(m);
    return r;
}

/* Reindex, gather form: score only the pooled positions (in pool order), select, map back */
int32_t orc_reindex_gather(const uint8_t* qc, const uint8_t* qs, const float* w, const uint8_t* kc,
                           const uint8_t* ks, int64_t n, const int32_t* pool_blocks, int32_t count,
                           int32_t block, int32_t k, int32_t* out) {
    int64_t slots = (int64_t)count * block;
    double* I = (double*)malloc(sizeof(double) * (size_t)(slots > 0 ? slots : 1));
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(slots > 0 ? slots : 1));
    for (int32_t i = 0; i < count; ++i)
        for (int32_t r = 0; r < block; ++r) {
            int64_t s = (int64_t)pool_blocks[i] * block + r;
            int64_t slot = (int64_t)i * block + r;
            pos[slot] = s;
            I[slot] = s < n ? orc_score(qc, qs, w, kc + s * 64, ks + s * 4, NULL, NULL) : -INFINITY;
        }
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t cnt = orc_topk(I, slots, k, sel);
    for (int32_t t = 0; t < k; ++t) out[t] = t < cnt ? (int32_t)pos[sel[t]] : -1;
    free(sel);
    free(pos);
    free(I);
    return cnt;
}

/* ------------------------------------------------------------------ batched decode step
 * One decode token's indexer work for nq independent sequences, threaded over sequences:
 * Full layer (score every visible entry, top-k, block max, pin, pool), then each Reindex layer
 * in mask form (full scores with its own q and w, masked to the pool, top-k).
 * k_codes/k_scales hold every sequence's cache rows; sequence t uses rows k_base[t]..+n[t]-1.
 * q: [nq][32][64] codes + [nq][32][4] scales; w: [nq][32]; reindex q/w: [L][nq][...].
 * out_topk [nq][k], out_pool [nq][topk_blocks], out_pool_n [nq], out_rtopk [L][nq][k].
 */
typedef struct {
    const uint8_t *kc, *ks;
    const int64_t* base;
    const int64_t* n;
    const uint8_t *qc, *qs, *rqc, *rqs;
    const float *w, *rw;
    int32_t nq, k, block, topk_blocks, layers;
    int32_t *out_topk, *out_pool, *out_pool_n, *out_rtopk;
    int32_t next;
    pthread_mutex_t mu;
} dec_ctx;

static void decode_one(dec_ctx* c, int32_t t) {
    int64_t n = c->n[t];
    const uint8_t* kc = c->kc + c->base[t] * 64;
    const uint8_t* ks = c->ks + c->base[t] * 4;
    double* I = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* bm = (double*)malloc(sizeof(double) * (size_t)(n / c->block + 2));
    orc_score_rows(c->qc + (int64_t)t * 32 * 64, c->qs + (int64_t)t * 32 * 4, c->w + (int64_t)t * 32, kc, ks, n, I,
                   NULL, NULL);
    orc_topk(I, n, c->k, c->out_topk + (int64_t)t * c->k);
    orc_block_max(I, n, c->block, bm);
    int32_t* pool = c->out_pool + (int64_t)t * c->topk_blocks;
    int32_t cnt = orc_pool(bm, n, c->block, c->topk_blocks, pool);
    c->out_pool_n[t] = cnt;
    for (int32_t l = 0; l < c->layers; ++l) {
        int64_t li = (int64_t)l * c->nq + t;
        orc_score_rows(c->rqc + li * 32 * 64, c->rqs + li * 32 * 4, c->rw + li * 32, kc, ks, n, I, NULL, NULL);
        orc_reindex_mask(I, n, pool, cnt, c->block, c->k, c->out_rtopk + li * c->k);
    }
    free(bm);
    free(I);
}

static void* decode_worker(void* p) {
    dec_ctx* c = (dec_ctx*)p;
    for (;;) {
        pthread_mutex_lock(&c->mu);
        int32_t t = c->next++;
        pthread_mutex_unlock(&c->mu);
        if (t >= c->nq) break;
        decode_one(c, t);
    }
    return NULL;
}

void orc_decode_batch(const uint8_t* kc, const uint8_t* ks, const int64_t* base, const int64_t* n, int32_t nq,
                      const uint8_t* qc, const uint8_t* qs, const float* w, int32_t layers, const uint8_t* rqc,
                      const uint8_t* rqs, const float* rw, int32_t k, int32_t block, int32_t topk_blocks,
                      int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, int32_t* out_rtopk, int nthreads) {
    dec_ctx c = {kc, ks, base, n, qc, qs, rqc, rqs, w, rw, nq, k, block, topk_blocks, layers,
                 out_topk, out_pool, out_pool_n, out_rtopk, 0, PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, decode_worker, &c);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------ main KV codec
 * [P1] "the scale format decides precision": 512-value rows, groups of 16 with an E4M3 scale,
 * no global scale ("removing the global scale still leaves enough range"): 256 + 32 bytes. */
#define MKV_DIM 512
#define MKV_GROUP 16

/* value of an E4M3 byte (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
 * subnormal m/8 * 2^-6; S.1111.111 is NaN) */
double orc_e4m3_value(int b) {
    const int sgn = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* byte of the smallest non-negative E4M3 value s with 6 * s >= a (a >= 0): the positive bytes
 * 0x00 .. 0x7e are in ascending value order; above 6 * 448 the largest (0x7e) */
int orc_e4m3_scale_for(double a) {
    for (int b = 0; b <= 0x7e; ++b)
        if (6.0 * orc_e4m3_value(b) >= a) return b;
    return 0x7e;
}

/* one 512-value row of bf16: codes[256] (element 2i in the low nibble of byte i), scales[32] */
void orc_mkv_quantize_row(const uint16_t* x, uint8_t* codes, uint8_t* scales) {
    for (int g = 0; g < MKV_DIM / MKV_GROUP; ++g) {
        double a = 0.0;
        for (int c = 0; c < MKV_GROUP; ++c) {
            const double v = fabs(bf16_value(x[g * MKV_GROUP + c]));
            if (v > a) a = v;
        }
        const int b = orc_e4m3_scale_for(a);
        const double sc = orc_e4m3_value(b);
        scales[g] = (uint8_t)b;
        for (int c = 0; c < MKV_GROUP; c += 2) {
            const int lo = sc > 0.0 ? orc_e2m1_code(bf16_value(x[g * MKV_GROUP + c]) / sc) : 0;
            const int hi = sc > 0.0 ? orc_e2m1_code(bf16_value(x[g * MKV_GROUP + c + 1]) / sc) : 0;
            codes[(g * MKV_GROUP + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

void orc_mkv_quantize_rows(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales) {
    for (int64_t r = 0; r < rows; ++r)
        orc_mkv_quantize_row(x + r * MKV_DIM, codes + r * (MKV_DIM / 2), scales + r * (MKV_DIM / MKV_GROUP));
}

/* value of element c of a stored row */
double orc_mkv_value(const uint8_t* codes, const uint8_t* scales, int c) {
    const int code = (codes[c / 2] >> (4 * (c & 1))) & 15;
    return orc_e2m1_value(code) * orc_e4m3_value(scales[c / MKV_GROUP]);
}

/* exact bf16 bit pattern of v; returns 0 and leaves *out untouched when v is not representable */
static int bf16_exact(double v, uint16_t* out) {
    const float f = (float)v;
    if ((double)f != v && !(isnan(v) && isnan(f))) return 0;
    uint32_t u;
    memcpy(&u, &f, 4);
    if (!isnan(f) && (u & 0xffffu) != 0) return 0;
    *out = isnan(f) ? (uint16_t)0x7fc0 : (uint16_t)(u >> 16);
    return 1;
}

/* gather-dequantise: out[t][i][0..511] = the bf16 values of row base[t] + idx[t][i] for
 * 0 <= idx[t][i] < n[t], zeros otherwise. Returns the number of values that were not exactly
 * representable in bf16 (0 for every E2M1 x E4M3 product). */
int64_t orc_mkv_gather(const uint8_t* codes, const uint8_t* scales, const int64_t* base, const int64_t* n,
                       const int32_t* idx, int32_t nq, int32_t k, int64_t idx_stride, uint16_t* out) {
    int64_t inexact = 0;
    for (int32_t t = 0; t < nq; ++t)
        for (int32_t i = 0; i < k; ++i) {
            const int64_t p = idx[t * idx_stride + i];
            uint16_t* o = out + ((int64_t)t * k + i) * MKV_DIM;
            if (p < 0 || p >= n[t]) {
                memset(o, 0, MKV_DIM * sizeof(uint16_t));
                continue;
            }
            const int64_t r = base[t] + p;
            for (int c = 0; c < MKV_DIM; ++c)
                if (!bf16_exact(orc_mkv_value(codes + r * (MKV_DIM / 2), scales + r * (MKV_DIM / MKV_GROUP), c),
                                &o[c]))
                    ++inexact;
        }
    return inexact;
}
