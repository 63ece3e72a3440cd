/*
 * Seeded synthetic inputs shared by the tests, the smoke check and the
 * benchmark.  This file draws random numbers and rounds them to bf16; it
 * holds none of the quantizer's arithmetic.
 *
 * Counter-based: element i of stream t in config c depends only on (c, t, i),
 *   h(c, t, i) = splitmix64(splitmix64(splitmix64(c) ^ t) ^ i),
 * so results do not depend on the thread count or on chunking.
 *   uniform  u(c,t,i) = (h >> 11) * 2^-53                         in [0, 1)
 *   normal   z(c,t,i) = sqrt(-2 ln(1 - u(c,t,2i))) cos(2 pi u(c,t,2i+1))
 *   student-t(3) = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), z_j = z(c,t,4i+j)
 * Values are rounded double -> binary32 -> bf16 (nearest-even at each step).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t hash3(uint64_t c, uint64_t t, uint64_t i) {
    return splitmix64(splitmix64(splitmix64(c) ^ t) ^ i);
}

static double unif(uint64_t c, uint64_t t, uint64_t i) {
    return (double)(hash3(c, t, i) >> 11) * 0x1.0p-53;
}

static double normal(uint64_t c, uint64_t t, uint64_t i) {
    double u1 = unif(c, t, 2 * i), u2 = unif(c, t, 2 * i + 1);
    return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
}

static double student_t3(uint64_t c, uint64_t t, uint64_t i) {
    double z0 = normal(c, t, 4 * i), z1 = normal(c, t, 4 * i + 1);
    double z2 = normal(c, t, 4 * i + 2), z3 = normal(c, t, 4 * i + 3);
    return z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
}

/* double -> binary32 (C cast, nearest-even) -> bf16 bits (nearest-even). */
static uint16_t to_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---- kinds of fill -------------------------------------------------------- */
enum { K_NORMAL = 0, K_OUT_UNIFORM = 1, K_OUT_T3 = 2, K_UNIFORM = 3 };

typedef struct {
    int kind;
    uint64_t c, t, t2;
    int64_t start, n;
    double a, b, p;
    uint16_t* out;     /* for fills */
    double* dout;      /* for K_UNIFORM */
} job_t;

static void run_range(const job_t* j, int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k) {
        uint64_t i = (uint64_t)(j->start + k);
        switch (j->kind) {
        case K_NORMAL: /* N(0, a^2) */
            j->out[k] = to_bf16(j->a * normal(j->c, j->t, i));
            break;
        case K_OUT_UNIFORM: /* with probability p: +-U[a, b] */
            if (unif(j->c, j->t, i) < j->p) {
                double mag = j->a + (j->b - j->a) * unif(j->c, j->t2, 2 * i + 1);
                double sgn = (hash3(j->c, j->t2, 2 * i) & 1) ? -1.0 : 1.0;
                j->out[k] = to_bf16(sgn * mag);
            }
            break;
        case K_OUT_T3: /* with probability p: a * t3 */
            if (unif(j->c, j->t, i) < j->p) j->out[k] = to_bf16(j->a * student_t3(j->c, j->t2, i));
            break;
        case K_UNIFORM:
            j->dout[k] = unif(j->c, j->t, i);
            break;
        }
    }
}

typedef struct {
    const job_t* job;
    int64_t lo, hi;
} slice_t;

static void* worker(void* arg) {
    slice_t* s = (slice_t*)arg;
    run_range(s->job, s->lo, s->hi);
    return NULL;
}

static void run(job_t* j, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (j->n < 65536 || nthreads == 1) {
        run_range(j, 0, j->n);
        return;
    }
    pthread_t th[64];
    slice_t sl[64];
    int created[64];
    int64_t per = (j->n + nthreads - 1) / nthreads;
    for (int k = 0; k < nthreads; ++k) {
        sl[k].job = j;
        sl[k].lo = k * per < j->n ? k * per : j->n;
        sl[k].hi = (k + 1) * per < j->n ? (k + 1) * per : j->n;
        created[k] = 0;
        if (sl[k].lo >= sl[k].hi) continue;
        if (pthread_create(&th[k], NULL, worker, &sl[k]) == 0) created[k] = 1;
        else run_range(j, sl[k].lo, sl[k].hi);
    }
    for (int k = 0; k < nthreads; ++k)
        if (created[k]) pthread_join(th[k], NULL);
}

void synth_normal_bf16(uint64_t c, uint64_t t, int64_t start, int64_t n, double sigma,
                       uint16_t* out, int nthreads) {
    job_t j = {K_NORMAL, c, t, 0, start, n, sigma, 0, 0, out, NULL};
    run(&j, nthreads);
}

void synth_outliers_uniform_bf16(uint64_t c, uint64_t t_mask, uint64_t t_val, int64_t start, int64_t n,
                                 double p, double lo, double hi, uint16_t* out, int nthreads) {
    job_t j = {K_OUT_UNIFORM, c, t_mask, t_val, start, n, lo, hi, p, out, NULL};
    run(&j, nthreads);
}

void synth_outliers_t3_bf16(uint64_t c, uint64_t t_mask, uint64_t t_val, int64_t start, int64_t n,
                            double p, double mult, uint16_t* out, int nthreads) {
    job_t j = {K_OUT_T3, c, t_mask, t_val, start, n, mult, 0, p, out, NULL};
    run(&j, nthreads);
}

void synth_uniform_f64(uint64_t c, uint64_t t, int64_t start, int64_t n, double* out, int nthreads) {
    job_t j = {K_UNIFORM, c, t, 0, start, n, 0, 0, 0, NULL, out};
    run(&j, nthreads);
}
