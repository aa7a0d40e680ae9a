/*
 * oracle.c -- plain, slow CPU reference of the routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * cpu_baseline leg load this library. The HIP library and its Python binding
 * never call it, and the two share no code: not the number formats, not the
 * plan, not any helper.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Round 4 Track C: Prefill MoE Plan (mm_clear + mm_hist + mm_scan +
 *       mm_place) & Epilogue / Gather Audit": section 1 (Executive Summary,
 *       findings 1, 2 and 4) and section 3 (Bitwise & Numerical Parity).
 *  [P3] "Batched resident MoE experts on Apple Silicon: a flat parallel expert
 *       pass": section 1 (Contribution) and section 3 (Results).
 *  [P4] "Add --moe-mode sweep-prefill: streamed expert supply for CPU
 *       mul_mat_id": Mechanism.
 *
 * Conventions: entry i = t*K + k (token-major). Floating point is decoded
 * exactly from its bit pattern and accumulated in double. No blocking,
 * fusion or reordering beyond the definitions written here.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): rows of one expert are ordered by entry index (stable); pad rows
 * carry token -1 and weight +0.0; the gate weight multiplies the down
 * projection's output; SwiGLU is silu(gate) * up with silu(z) = z/(1+e^-z);
 * ids equal to -1 are skipped and any other id outside [0, E) is counted as
 * bad and skipped.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

/* ------------------------------------------------------------------------- */
/* Number formats, from the IEEE 754 binary16 definition and from bfloat16    */
/* being the upper half of an IEEE binary32.                                   */
/* ------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)m, -24);                  /* subnormal: m * 2^-24 */
    else if (ex == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), ex - 25);     /* 1.m * 2^(ex-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to binary16, to nearest with ties to even (nearbyint in the
 * default rounding mode), with gradual underflow and overflow to infinity. */
uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (isinf(v))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {                      /* subnormal range: q * 2^-24 */
        double q = nearbyint(ldexp(a, 24));         /* q == 1024 is the smallest normal */
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);                                  /* a = fr * 2^e2, fr in [0.5, 1) */
    int E = e2 - 1;                                 /* a = 1.xxx * 2^E */
    double q = nearbyint(ldexp(a, 10 - E));         /* 10 fraction bits: q in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0);
}

/* Round a double to bfloat16 (8 exponent bits, bias 127, 7 fraction bits),
 * to nearest with ties to even, gradual underflow, overflow to infinity. */
uint16_t oracle_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7fc0;
    if (isinf(v))
        return sign | 0x7f80;
    if (a < ldexp(1.0, -126)) {                     /* subnormal range: q * 2^-133 */
        double q = nearbyint(ldexp(a, 133));
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    double q = nearbyint(ldexp(a, 7 - E));          /* q in [128, 256] */
    if (q == 256.0) {
        q = 128.0;
        E += 1;
    }
    if (E > 127)
        return sign | 0x7f80;
    return sign | (uint16_t)((E + 127) << 7) | (uint16_t)(q - 128.0);
}

void oracle_f16_to_f64_n(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}
void oracle_bf16_to_f64_n(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}
void oracle_f64_to_f16_n(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(in[i]);
}
void oracle_f64_to_bf16_n(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(in[i]);
}

/* Exact decode table for binary16 (all 65536 patterns), filled once. */
static double f16_table[65536];
static int f16_table_ready = 0;

static void init_tables(void)
{
    if (f16_table_ready)
        return;
    for (int h = 0; h < 65536; ++h) f16_table[h] = oracle_f16_to_f64((uint16_t)h);
    f16_table_ready = 1;
}

/* element j of an array of the given element type, as a double */
static double elem(const void *p, int dtype, size_t j)
{
    if (dtype == OR_F32)
        return (double)((const float *)p)[j];
    if (dtype == OR_F16)
        return f16_table[((const uint16_t *)p)[j]];
    return oracle_bf16_to_f64(((const uint16_t *)p)[j]);
}

/* the value v rounded to the element type and decoded back */
static double round_to(double v, int dtype)
{
    if (dtype == OR_F32)
        return (double)(float)v;
    if (dtype == OR_F16)
        return oracle_f16_to_f64(oracle_f64_to_f16(v));
    return oracle_bf16_to_f64(oracle_f64_to_bf16(v));
}

/* ------------------------------------------------------------------------- */
/* Routing plan: a counting sort of the (token, k) entries by expert.          */
/* ------------------------------------------------------------------------- */

/* meta[] fields */
enum { M_NENT, M_NBLK, M_NR, M_NT, M_NACTIVE, M_MAXCNT, M_NSKIP, M_NBAD, M_TM, M_E, M_K, M_N };

/*
 * [P1] s.1 findings 1-2: a per-expert count over all entries; each expert's
 * count is padded up to a multiple of tm and the padded counts are laid out
 * back to back in ascending expert order ([P4] Mechanism: experts are visited
 * in ascending id order over contiguous slices); every entry goes to the row
 * equal to its expert's start plus the number of earlier entries with the same
 * expert (the in-block rank plus the block offset, which adds up to exactly
 * that); the pad rows at the end of each expert's range get token -1.
 * [P1] s.3 lists the outputs compared: meta, boff, eoff, tiles, stok, sw, pos.
 *
 * Outputs: cnt[E], eoff[E+1], tiles[nt], stok[nr], sw[nr], pos[T*K],
 * meta[11], and boff[nblk*E] if boff != NULL, where a block is B consecutive
 * entries. Returns 0, or -1 on bad arguments.
 */
int oracle_plan(const int32_t *ids, const float *w, int64_t T, int K, int E, int tm, int B,
                int32_t *cnt, int32_t *eoff, int32_t *tiles, int32_t *stok, float *sw,
                int32_t *pos, int32_t *meta, int32_t *boff)
{
    if (T < 1 || K < 1 || E < 1 || tm < 1 || B < 1)
        return -1;
    int64_t nent = T * K;
    int64_t nskip = 0, nbad = 0;

    /* 1. histogram; -1 means skipped, anything else outside [0,E) is bad */
    for (int e = 0; e < E; ++e) cnt[e] = 0;
    for (int64_t i = 0; i < nent; ++i) {
        int e = ids[i];
        if (e == -1)
            nskip++;
        else if (e < 0 || e >= E)
            nbad++;
        else
            cnt[e]++;
    }

    /* 2. rows_e = cnt_e rounded up to tm; eoff = exclusive prefix sum over e */
    eoff[0] = 0;
    for (int e = 0; e < E; ++e) {
        int64_t rows = ((int64_t)cnt[e] + tm - 1) / tm * tm;
        eoff[e + 1] = (int32_t)(eoff[e] + rows);
    }
    int64_t nr = eoff[E];

    /* 3. tiles: the expert of each tm-row tile */
    for (int e = 0; e < E; ++e)
        for (int64_t j = eoff[e] / tm; j < eoff[e + 1] / tm; ++j) tiles[j] = e;

    /* 4. stable placement: entries of expert e in ascending entry order */
    int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    if (!fill)
        return -1;
    for (int e = 0; e < E; ++e) fill[e] = eoff[e];
    for (int64_t i = 0; i < nent; ++i) {
        int e = ids[i];
        if (e < 0 || e >= E) {
            pos[i] = -1;
            continue;
        }
        int64_t r = fill[e]++;
        stok[r] = (int32_t)(i / K);
        sw[r] = w[i];               /* bit copy */
        pos[i] = (int32_t)r;
    }
    free(fill);

    /* 5. pad rows */
    for (int e = 0; e < E; ++e)
        for (int64_t r = eoff[e] + cnt[e]; r < eoff[e + 1]; ++r) {
            stok[r] = -1;
            sw[r] = 0.0f;
        }

    /* 6. meta */
    int64_t nactive = 0, maxcnt = 0;
    for (int e = 0; e < E; ++e) {
        if (cnt[e] > 0)
            nactive++;
        if (cnt[e] > maxcnt)
            maxcnt = cnt[e];
    }
    int64_t nblk = (nent + B - 1) / B;
    meta[M_NENT] = (int32_t)nent;
    meta[M_NBLK] = (int32_t)nblk;
    meta[M_NR] = (int32_t)nr;
    meta[M_NT] = (int32_t)(nr / tm);
    meta[M_NACTIVE] = (int32_t)nactive;
    meta[M_MAXCNT] = (int32_t)maxcnt;
    meta[M_NSKIP] = (int32_t)nskip;
    meta[M_NBAD] = (int32_t)nbad;
    meta[M_TM] = tm;
    meta[M_E] = E;
    meta[M_K] = K;

    /* 7. optional: boff[b][e] = entries of expert e in the blocks before b */
    if (boff) {
        int64_t *run = (int64_t *)calloc((size_t)E, sizeof(int64_t));
        if (!run)
            return -1;
        for (int64_t b = 0; b < nblk; ++b) {
            for (int e = 0; e < E; ++e) boff[b * E + e] = (int32_t)run[e];
            for (int64_t i = b * B; i < nent && i < (b + 1) * B; ++i) {
                int e = ids[i];
                if (e >= 0 && e < E)
                    run[e]++;
            }
        }
        free(run);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gather: [P1] s.1 finding 4 -- each routed row is a bit copy of its token's  */
/* half-precision row. Pad rows (token -1) are all-zero bits.                  */
/* ------------------------------------------------------------------------- */
void oracle_gather(const void *x, int elem_bytes, int64_t T, int d, const int32_t *stok,
                   int64_t nr, void *xs)
{
    size_t rb = (size_t)d * (size_t)elem_bytes;
    for (int64_t r = 0; r < nr; ++r) {
        char *dst = (char *)xs + (size_t)r * rb;
        int t = stok[r];
        if (t >= 0 && t < T)
            memcpy(dst, (const char *)x + (size_t)t * rb, rb);
        else
            memset(dst, 0, rb);
    }
}

/* ------------------------------------------------------------------------- */
/* Expert FFN, the naive per-(token, expert) loop of [P3] s.1: for one token   */
/* and one of its experts, gate and up projections, gated activation, down     */
/* projection. All in double; with round_h the activation h is rounded to the  */
/* element type first, as the fp16-operand reference of [P1] s.3 does.        */
/* ------------------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y[c] = sum_j h[j] * Wd[e][j][c], h[j] = silu(g[j]) * u[j],
 * g[j] = sum_i x[t][i] * Wg[e][i][j], u[j] = sum_i x[t][i] * Wu[e][i][j].
 * g, u, h: caller scratch of f doubles. */
static void ffn_one(const void *x, int64_t t, int e, const void *wg, const void *wu, const void *wd,
                    int dtype, int d, int f, int round_h, double *g, double *u, double *h, double *y)
{
    size_t xo = (size_t)t * d;
    size_t wo = (size_t)e * d * f;
    for (int j = 0; j < f; ++j) g[j] = u[j] = 0.0;
    for (int i = 0; i < d; ++i) {
        double xi = elem(x, dtype, xo + i);
        for (int j = 0; j < f; ++j) {
            g[j] += xi * elem(wg, dtype, wo + (size_t)i * f + j);
            u[j] += xi * elem(wu, dtype, wo + (size_t)i * f + j);
        }
    }
    for (int j = 0; j < f; ++j) {
        h[j] = silu(g[j]) * u[j];
        if (round_h)
            h[j] = round_to(h[j], dtype);
    }
    for (int c = 0; c < d; ++c) y[c] = 0.0;
    for (int j = 0; j < f; ++j)
        for (int c = 0; c < d; ++c) y[c] += h[j] * elem(wd, dtype, wo + (size_t)j * d + c);
}

/*
 * Layer output of the listed tokens: out[q][c] = sum over k = 0..K-1 (in that
 * order, [P3] s.3: a fixed per-token top-k summation order) of
 * w[t][k] * FFN_{ids[t][k]}(x[t]) with t = tok[q], skipping ids outside
 * [0, E); the weight multiplies the expert output ([P3] s.1: weighted down
 * projection). Double throughout; the caller rounds to fp32.
 * OpenMP over the listed tokens (each is independent).
 */
int oracle_ffn(const void *x, const int32_t *ids, const float *w, const void *wg, const void *wu,
               const void *wd, int dtype, int64_t T, int K, int E, int d, int f, int round_h,
               const int32_t *tok, int64_t ntok, double *out, int nthreads)
{
    if (d < 1 || f < 1 || K < 1 || E < 1)
        return -1;
    init_tables();
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t q = 0; q < ntok; ++q) {
        double *g = (double *)malloc(sizeof(double) * (size_t)(3 * f + 2 * d));
        if (!g) {
            fail = 1;
            continue;
        }
        double *u = g + f, *h = u + f, *y = h + f, *acc = y + d;
        int64_t t = tok[q];
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        if (t >= 0 && t < T) {
            for (int k = 0; k < K; ++k) {
                int e = ids[t * K + k];
                if (e < 0 || e >= E)
                    continue;
                ffn_one(x, t, e, wg, wu, wd, dtype, d, f, round_h, g, u, h, y);
                double wk = (double)w[t * K + k];
                for (int c = 0; c < d; ++c) acc[c] += wk * y[c];
            }
        }
        for (int c = 0; c < d; ++c) out[q * d + c] = acc[c];
        free(g);
    }
    return fail ? -1 : 0;
}

/*
 * Per-entry expert outputs: for entry i = ent[q] (token t = i / K, expert
 * e = ids[i] in [0, E)), y[q][c] = w[i] * FFN_e(x[t])[c] and h[q][j] = the
 * activation fed to the down projection (rounded as round_h says).
 * Entries with an id outside [0, E) give zero rows.
 */
int oracle_ffn_entries(const void *x, const int32_t *ids, const float *w, const void *wg,
                       const void *wu, const void *wd, int dtype, int64_t T, int K, int E, int d,
                       int f, int round_h, const int32_t *ent, int64_t nq, double *y, double *h_out,
                       int nthreads)
{
    if (d < 1 || f < 1 || K < 1 || E < 1)
        return -1;
    init_tables();
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t q = 0; q < nq; ++q) {
        double *g = (double *)malloc(sizeof(double) * (size_t)(3 * f + d));
        if (!g) {
            fail = 1;
            continue;
        }
        double *u = g + f, *h = u + f, *yy = h + f;
        int64_t i = ent[q];
        int e = (i >= 0 && i < T * K) ? ids[i] : -1;
        if (e >= 0 && e < E) {
            ffn_one(x, i / K, e, wg, wu, wd, dtype, d, f, round_h, g, u, h, yy);
            double wi = (double)w[i];
            for (int c = 0; c < d; ++c) y[q * d + c] = wi * yy[c];
            if (h_out)
                for (int j = 0; j < f; ++j) h_out[q * f + j] = h[j];
        } else {
            for (int c = 0; c < d; ++c) y[q * d + c] = 0.0;
            if (h_out)
                for (int j = 0; j < f; ++j) h_out[q * f + j] = 0.0;
        }
        free(g);
    }
    return fail ? -1 : 0;
}

/*
 * Brute force for tiny inputs: evaluate every expert on every token, then mask
 * by the router's choice: out[t] = sum_e m[t][e] * FFN_e(x[t]) with
 * m[t][e] = sum_k [ids[t][k] == e] * w[t][k]. Experts in ascending order.
 */
int oracle_dense_masked(const void *x, const int32_t *ids, const float *w, const void *wg,
                        const void *wu, const void *wd, int dtype, int64_t T, int K, int E, int d,
                        int f, int round_h, double *out)
{
    init_tables();
    double *g = (double *)malloc(sizeof(double) * (size_t)(3 * f + d + E));
    if (!g)
        return -1;
    double *u = g + f, *h = u + f, *y = h + f, *m = y + d;
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) m[e] = 0.0;
        for (int k = 0; k < K; ++k) {
            int e = ids[t * K + k];
            if (e >= 0 && e < E)
                m[e] += (double)w[t * K + k];
        }
        for (int c = 0; c < d; ++c) out[t * d + c] = 0.0;
        for (int e = 0; e < E; ++e) {
            ffn_one(x, t, e, wg, wu, wd, dtype, d, f, round_h, g, u, h, y);
            for (int c = 0; c < d; ++c) out[t * d + c] += m[e] * y[c];
        }
    }
    free(g);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Combine in fp32: out[t][c] = +0.0f, then += Y[pos[t*K+k]][c] for k = 0..K-1 */
/* in that order ([P3] s.3), skipping pos < 0. One correct fp32 result.       */
/* ------------------------------------------------------------------------- */
void oracle_combine_f32(const float *Y, const int32_t *pos, int64_t T, int K, int d, float *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = pos[t * K + k];
                if (r >= 0)
                    acc = acc + Y[(size_t)r * d + c];
            }
            out[t * d + c] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Compact expert outputs (a storage format of the layer's intermediate y,    */
/* not a step of the pages): each row is cut into blocks of 128 columns (the  */
/* last one may be shorter); a block holds binary16 values s[c] and one       */
/* exponent e and stands for the values s[c] * 2^-e, exactly.                 */
/* Encoding of fp32 values v[c]: M = the largest |v[c]| of the block (NaN     */
/* ignored). If M is 0 or not finite, e = 0. Otherwise M = m * 2^k with m in  */
/* [1/2, 1) and e = 15 - k, clamped to [-112, 100], so that M * 2^e lies in   */
/* [2^14, 2^15). s[c] = v[c] * 2^e rounded to binary16, nearest even. The     */
/* scaling by 2^e is exact, and over that range of e every decoded binary16   */
/* value is an exact fp32 number.                                             */
/* ------------------------------------------------------------------------- */
#define Y16_BLOCK 128

int oracle_y16_exponent(float M)
{
    if (!(M > 0.0f) || isinf(M))
        return 0;
    int k;
    frexp((double)M, &k);
    int e = 15 - k;
    return e < -112 ? -112 : (e > 100 ? 100 : e);
}

void oracle_y16_encode(const float *y, int64_t nrows, int d, uint16_t *s, int8_t *ex)
{
    int nb = (d + Y16_BLOCK - 1) / Y16_BLOCK;
    for (int64_t r = 0; r < nrows; ++r)
        for (int b = 0; b < nb; ++b) {
            int c0 = b * Y16_BLOCK, c1 = c0 + Y16_BLOCK < d ? c0 + Y16_BLOCK : d;
            float M = 0.0f;
            for (int c = c0; c < c1; ++c) M = fmaxf(M, fabsf(y[(size_t)r * d + c]));
            int e = oracle_y16_exponent(M);
            ex[(size_t)r * nb + b] = (int8_t)e;
            for (int c = c0; c < c1; ++c)
                s[(size_t)r * d + c] = oracle_f64_to_f16(ldexp((double)y[(size_t)r * d + c], e));
        }
}

void oracle_y16_decode(const uint16_t *s, const int8_t *ex, int64_t nrows, int d, float *y)
{
    int nb = (d + Y16_BLOCK - 1) / Y16_BLOCK;
    for (int64_t r = 0; r < nrows; ++r)
        for (int c = 0; c < d; ++c)
            y[(size_t)r * d + c] = (float)ldexp(oracle_f16_to_f64(s[(size_t)r * d + c]),
                                                -(int)ex[(size_t)r * nb + c / Y16_BLOCK]);
}

/* The combine over compact rows: each value decoded exactly, then the same   */
/* fp32 sum from +0.0f in k order as oracle_combine_f32.                      */
void oracle_combine_y16(const uint16_t *s, const int8_t *ex, const int32_t *pos, int64_t T, int K,
                        int d, float *out)
{
    int nb = (d + Y16_BLOCK - 1) / Y16_BLOCK;
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = pos[t * K + k];
                if (r >= 0)
                    acc = acc + (float)ldexp(oracle_f16_to_f64(s[(size_t)r * d + c]),
                                             -(int)ex[(size_t)r * nb + c / Y16_BLOCK]);
            }
            out[t * d + c] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Router: [P1] s.1 finding 5 and s.3 name the kernel that writes the routed  */
/* ids (route_topk); the workload description fixes what it computes: a      */
/* softmax over the E router logits, the K largest probabilities kept and     */
/* renormalised to sum to one. Since softmax is monotone, the K largest       */
/* probabilities are the K largest logits, and the renormalised weight of     */
/* pick k is exp(l_k - m) / sum over the K picks of exp(l_j - m), m = the     */
/* largest logit (the full softmax denominator cancels).                      */
/* Order: descending logit, equal logits by ascending expert id. NaN logits   */
/* are never picked; if fewer than K logits are not NaN, the remaining picks  */
/* are id -1 with weight 0.                                                   */
/* ------------------------------------------------------------------------- */
int oracle_route_topk(const float *logits, int64_t T, int E, int K, int32_t *ids, double *w)
{
    if (T < 1 || E < 1 || K < 1)
        return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e) taken[e] = isnan(l[e]) ? 1 : 0;
        int n = 0;
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e)  /* first index wins ties */
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            ids[t * K + k] = best;
            if (best >= 0) {
                taken[best] = 1;
                n++;
            }
        }
        double m = n > 0 ? (double)l[ids[t * K]] : 0.0, sum = 0.0;
        for (int k = 0; k < n; ++k) sum += exp((double)l[ids[t * K + k]] - m);
        for (int k = 0; k < K; ++k)
            w[t * K + k] = k < n ? exp((double)l[ids[t * K + k]] - m) / sum : 0.0;
    }
    free(taken);
    return 0;
}
