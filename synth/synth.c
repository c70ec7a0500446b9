/*
 * Seeded synthetic inputs for the FP4 lightning indexer (input generation only).
 *
 * This module produces the raw inputs that both the CPU oracle and the GPU path consume:
 * bf16 query and key vectors, fp32 head weights, the +-1 sign vector of the random Hadamard
 * rotation, per-sequence lengths and the planted high-score key positions. It contains none
 * of the method's arithmetic (no rotation, quantisation, scoring or selection).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014), used as a counter-based generator: value i of stream
 * (seed, tag, sub) is mix64(s0 + (i + 1) * GOLDEN), where s0 is derived from the triple by
 * mixing. Normals come from Box-Muller in fp64 (cosine branch only, so normal i uses uniforms
 * 2i and 2i+1) and are rounded to bf16 with round-to-nearest-even.
 *
 * Workload recipe (the pages fix 32 heads x 128 dims, FP4 q and k, fp32 weights):
 *   q ~ N(0,1) per element, k ~ N(0,1) per element, w ~ N(0, 1/32),
 *   about 1% of keys per sequence shifted by 0.5 x (mean over heads of the query).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_stream(uint64_t seed, uint64_t tag, uint64_t sub) {
    return mix64(mix64(seed + 0xA0761D6478BD642Full) + tag * GOLDEN + mix64(sub ^ 0xE7037ED1A0B428DBull));
}

static inline uint64_t draw(uint64_t s0, uint64_t i) { return mix64(s0 + (i + 1) * GOLDEN); }

/* uniform in [0, 1) with 53 random bits */
static inline double unif(uint64_t s0, uint64_t i) { return (double)(draw(s0, i) >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t s0, uint64_t i) {
    double u1 = unif(s0, 2 * i), u2 = unif(s0, 2 * i + 1);
    return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
}

/* round an fp64 value to bf16 (8 significant bits), nearest-even; returns the bf16 bit pattern */
uint16_t synth_bf16_rne(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
    int e;
    double m = frexp(x, &e);             /* x = m * 2^e, 0.5 <= |m| < 1 */
    double r = rint(ldexp(m, 8));         /* 8 significant bits, ties to even (default mode) */
    float f = (float)ldexp(r, e - 8);     /* exactly representable in fp32 for our ranges */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

double synth_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double synth_uniform(uint64_t seed, uint64_t tag, uint64_t sub, uint64_t i) {
    return unif(synth_stream(seed, tag, sub), i);
}

/* ---- threaded fill of bf16 normals ---- */
typedef struct {
    uint64_t s0, start, count;
    uint16_t* out;
} job_bf16;

static void* run_bf16(void* p) {
    job_bf16* j = (job_bf16*)p;
    for (uint64_t i = 0; i < j->count; ++i) j->out[i] = synth_bf16_rne(normal_at(j->s0, j->start + i));
    return NULL;
}

/* out[i] = bf16(N(0,1) draw number start+i of stream (seed, tag, sub)) */
void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t sub, uint64_t start, uint64_t count,
                       uint16_t* out, int nthreads) {
    uint64_t s0 = synth_stream(seed, tag, sub);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (count < 65536 || nthreads == 1) {
        job_bf16 j = {s0, start, count, out};
        run_bf16(&j);
        return;
    }
    pthread_t th[64];
    job_bf16 jobs[64];
    uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t b = per * (uint64_t)t;
        if (b >= count) break;
        uint64_t c = count - b < per ? count - b : per;
        jobs[t].s0 = s0; jobs[t].start = start + b; jobs[t].count = c; jobs[t].out = out + b;
        pthread_create(&th[t], NULL, run_bf16, &jobs[t]);
        ++used;
    }
    for (int t = 0; t < used; ++t) pthread_join(th[t], NULL);
}

/* out[i] = fp32(scale * N(0,1) draw start+i), rounded to nearest-even */
void synth_normal_f32(uint64_t seed, uint64_t tag, uint64_t sub, uint64_t start, uint64_t count,
                      double scale, float* out) {
    uint64_t s0 = synth_stream(seed, tag, sub);
    for (uint64_t i = 0; i < count; ++i) out[i] = (float)(scale * normal_at(s0, start + i));
}

/* sign vector of the random Hadamard rotation: +1 or -1 from the low bit of each draw */
void synth_signs(uint64_t seed, uint64_t tag, int8_t* out, int n) {
    uint64_t s0 = synth_stream(seed, tag, 0);
    for (int c = 0; c < n; ++c) out[c] = (draw(s0, (uint64_t)c) & 1u) ? (int8_t)-1 : (int8_t)1;
}

/* lengths: out[b] = lo + floor(u_b * span) */
void synth_lengths(uint64_t seed, uint64_t tag, int32_t nseq, int64_t lo, int64_t span, int64_t* out) {
    uint64_t s0 = synth_stream(seed, tag, 0);
    for (int32_t b = 0; b < nseq; ++b) {
        int64_t v = (int64_t)floor(unif(s0, (uint64_t)b) * (double)span);
        if (v >= span) v = span - 1;
        out[b] = lo + v;
    }
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* m distinct positions in [0, n), sorted ascending; Floyd's sampling without replacement
 * (Bentley and Floyd, "A sample of brilliance", CACM 1987). Returns m, or -1 on bad input. */
int64_t synth_plant_positions(uint64_t seed, uint64_t tag, uint64_t sub, int64_t n, int64_t m, int64_t* out) {
    if (n < 0 || m < 0 || m > n) return -1;
    if (m == 0) return 0;
    uint8_t* taken = (uint8_t*)calloc((size_t)((n + 7) / 8), 1);
    if (!taken) return -1;
    uint64_t s0 = synth_stream(seed, tag, sub);
    int64_t cnt = 0;
    for (int64_t j = n - m; j < n; ++j) {
        int64_t t = (int64_t)floor(unif(s0, (uint64_t)(j - (n - m))) * (double)(j + 1));
        if (t > j) t = j;
        if (taken[t >> 3] & (1u << (t & 7))) t = j;
        taken[t >> 3] |= (uint8_t)(1u << (t & 7));
        out[cnt++] = t;
    }
    free(taken);
    qsort(out, (size_t)cnt, sizeof(int64_t), cmp_i64);
    return cnt;
}

/* rows[r*128 + c] <- bf16(rows[r*128 + c] + shift[c]) for every r with pos[p] - row0 == r */
void synth_apply_plant(uint16_t* rows, int64_t row0, int64_t nrows, const int64_t* pos, int64_t npos,
                       const double* shift) {
    for (int64_t p = 0; p < npos; ++p) {
        int64_t r = pos[p] - row0;
        if (r < 0 || r >= nrows) continue;
        uint16_t* row = rows + r * 128;
        for (int c = 0; c < 128; ++c) row[c] = synth_bf16_rne(synth_bf16_to_double(row[c]) + shift[c]);
    }
}

/* shift[c] = 0.5 * mean over 32 heads of q[j*128 + c] (bf16 query of one position) */
void synth_plant_shift(const uint16_t* q, double* shift) {
    for (int c = 0; c < 128; ++c) {
        double s = 0.0;
        for (int j = 0; j < 32; ++j) s += synth_bf16_to_double(q[j * 128 + c]);
        shift[c] = 0.5 * (s / 32.0);
    }
}
