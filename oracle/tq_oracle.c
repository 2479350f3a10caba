/*
 * tq_oracle.c -- plain, slow CPU oracle of the turbo3 / turbo2 KV-cache block
 * codec.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
 * CPU-baseline leg may load it; the product path (the HIP library) must never
 * call, link or include anything from here, and this file includes nothing of
 * the product's.
 *
 * Source of the method: "llama.cpp に TurboQuant を実装 -- 2bit・3bit の KV
 * キャッシュ圧縮" (openalchemy.io blog):
 *   - section "TurboQuant の何が違うのか": rotate each vector by an orthogonal
 *     matrix before quantising, then a per-coordinate Lloyd-Max scalar
 *     quantiser; the rotation is undone on read; the fork replaces the dense
 *     rotation by a fast Walsh-Hadamard transform made only of additions and
 *     subtractions, which is its own inverse, so decode runs the same
 *     transform again and the scale can be folded elsewhere;
 *   - section "どこまで小さくなるのか": one block packs 128 values plus one FP16
 *     norm, 0.39 B/value for turbo3 and 0.27 B/value for turbo2;
 *   - section "実モデルでの数値": a head_dim of 256 is two stacked 128-blocks;
 *   - section "現在の実装と、これから": the cache is stored compressed and
 *     dequantised to FP16 before attention; a CPU reference path exists for
 *     correctness.
 * Where the page is silent the plainest reading is taken (each one is listed
 * beside the function that takes it).
 *
 * Arithmetic: IEEE binary64 throughout, scalar loops, no vector intrinsics,
 * built without -ffast-math and with floating-point contraction off.  Threads
 * only split independent blocks / rows.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "tq_oracle.h"

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16, written from the definition of the format.            */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 = zero / subnormal (f * 2^-24), 31 = inf / NaN. */
double tqo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round to nearest, ties to even.  The scaled significand is exact in double
 * and nearbyint() rounds it in the default (to-nearest-even) mode. */
uint16_t tqo_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (isinf(x))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m in [0, 1024] (1024 is the
         * smallest normal, whose bit pattern is the same integer). */
        double m = nearbyint(a * ldexp(1.0, 24));
        return sign | (uint16_t)m;
    }
    int e;
    double f = frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
    double m = nearbyint(f * 2048.0);  /* significand with 11 bits, [1024, 2048] */
    int E = e - 1;                     /* a ~ (m / 1024) * 2^E */
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0);
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max scalar quantiser for N(0,1).                                   */
/* ------------------------------------------------------------------------ */

static double std_pdf(double x) { return exp(-0.5 * x * x) / sqrt(8.0 * atan(1.0)); }
static double std_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Reading: the page asks for the optimal Lloyd-Max codebook of the rotated
 * coordinates and names no distribution; the rotated, normalised
 * coordinates are taken as N(0,1) (the levels +-0.4528/+-1.510 and
 * +-0.2451/+-0.7560/+-1.344/+-2.152 are the Gaussian ones).
 *
 * Lloyd's two optimality conditions, iterated to a fixed point:
 *   (1) each decision threshold is the midpoint of its two neighbouring levels;
 *   (2) each level is the mean of N(0,1) over its cell,
 *       E[X | a < X <= b] = (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)).
 * The density is symmetric, so the solution is too: the iteration runs on the
 * positive half-line with the middle threshold held at exactly 0 (for one bit
 * the single threshold is 0).  Levels come out ascending: code k <-> levels[k].
 * Returns the number of iterations, or -1 if it did not converge. */
int tqo_codebook(int bits, double *levels, double *thresholds)
{
    if (bits < 1 || bits > 4)
        return -1;
    int L = 1 << bits, P = L / 2;
    double pos[8], edge[9];
    /* start from evenly spaced positive levels */
    for (int k = 0; k < P; ++k)
        pos[k] = (k + 0.5) * (3.0 / P);
    int it;
    for (it = 1; it <= 100000; ++it) {
        edge[0] = 0.0;
        for (int k = 1; k < P; ++k)
            edge[k] = 0.5 * (pos[k - 1] + pos[k]);        /* condition (1) */
        double delta = 0.0;
        for (int k = 0; k < P; ++k) {
            double a = edge[k];
            double num, den;
            if (k == P - 1) {                              /* last cell is (a, inf) */
                num = std_pdf(a);
                den = 0.5 * erfc(a / sqrt(2.0));
            } else {
                double b = edge[k + 1];
                num = std_pdf(a) - std_pdf(b);
                den = std_cdf(b) - std_cdf(a);
            }
            double c = num / den;                          /* condition (2) */
            double d = fabs(c - pos[k]);
            if (d > delta)
                delta = d;
            pos[k] = c;
        }
        if (delta < 1e-15)
            break;
    }
    if (it > 100000)
        return -1;
    for (int k = 0; k < P; ++k) {
        levels[P + k] = pos[k];
        levels[P - 1 - k] = -pos[k];
    }
    for (int k = 0; k < L - 1; ++k)
        thresholds[k] = 0.5 * (levels[k] + levels[k + 1]);
    thresholds[P - 1] = 0.0; /* exactly; the midpoint of +-c is 0 */
    return it;
}

/* ------------------------------------------------------------------------ */
/* The rotation: fast Walsh-Hadamard transform over 128 values.             */
/* ------------------------------------------------------------------------ */

/* Reading: the page's transform is orthogonal, made of additions and
 * subtractions only, and is its own inverse.  The butterflies compute the unnormalised Sylvester Hadamard
 * matrix H (H[i][j] = (-1)^popcount(i & j), natural order), H*H = 128*I; the
 * orthonormal rotation is H / sqrt(128), whose scale the codec folds into the
 * norm.  No random sign flips (decode runs the very same transform). */
void tqo_fwht128(double *v)
{
    for (int h = 1; h < TQO_BLOCK; h <<= 1)
        for (int i = 0; i < TQO_BLOCK; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

/* ------------------------------------------------------------------------ */
/* One block: encode and decode.                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    int bits;
    double levels[16];
    double thr[15];
} codebook_t;

static int get_codebook(int bits, codebook_t *cb)
{
    if (bits != 2 && bits != 3)
        return -1;
    cb->bits = bits;
    return tqo_codebook(bits, cb->levels, cb->thr) < 0 ? -1 : 0;
}

/* Bit layout reading (the page fixes only the byte count): the 128 codes of a
 * block form one little-endian bit stream, code i at stream bits
 * [bits*i, bits*i + bits), least significant bit first; stream bit p lives in
 * byte p / 8 at bit p % 8.  16*bits bytes per block. */
static void pack_codes(int bits, const int *code, uint8_t *field)
{
    memset(field, 0, (size_t)(16 * bits));
    for (int i = 0; i < TQO_BLOCK; ++i)
        for (int j = 0; j < bits; ++j) {
            int p = bits * i + j;
            if ((code[i] >> j) & 1)
                field[p / 8] |= (uint8_t)(1u << (p % 8));
        }
}

static void unpack_codes(int bits, const uint8_t *field, int *code)
{
    for (int i = 0; i < TQO_BLOCK; ++i) {
        int c = 0;
        for (int j = 0; j < bits; ++j) {
            int p = bits * i + j;
            c |= ((field[p / 8] >> (p % 8)) & 1) << j;
        }
        code[i] = c;
    }
}

/* Encode steps, in the page's order:
 *   1. n = ||x||_2 of the 128 values (the FP16 norm the block keeps);
 *   2. rotate: u = H x, or u = H D x when a diagonal d of +-1 is given (the
 *      randomised Hadamard rotation: TurboQuant's rotation is a random
 *      orthogonal one, "何が違う"; H D is orthogonal up to the factor sqrt(128)
 *      for any signs, so the norm and the normalisation are unchanged);
 *   3. normalise: t = u / n, so that sum t_i^2 = 128 (unit mean square, the
 *      scale the N(0,1) codebook expects); the unrounded norm is used, only
 *      its stored copy is rounded;
 *   4. Lloyd-Max: code_i = number of thresholds tau_k with t_i >= tau_k
 *      (a value exactly on a threshold goes to the upper cell; -0.0 >= 0);
 *   5. pack the codes; store n16 = fp16_RNE(min(n, 65504)) (saturating).
 * Zero block (n == 0): t = 0, so every code is the first level above 0
 * (2^bits / 2), n16 = 0, and it decodes to exactly 0.
 * dist (optional, 128 doubles): min_k |t_i - tau_k|, for tie analysis. */
static void encode_block(const codebook_t *cb, const uint16_t *xh, uint8_t *field,
                         uint16_t *n16, double *dist, const double *d)
{
    double x[TQO_BLOCK], u[TQO_BLOCK];
    int code[TQO_BLOCK];
    int nthr = (1 << cb->bits) - 1;

    double ss = 0.0;
    for (int i = 0; i < TQO_BLOCK; ++i) {
        x[i] = tqo_half_to_double(xh[i]);
        ss += x[i] * x[i];
    }
    double n = sqrt(ss);

    for (int i = 0; i < TQO_BLOCK; ++i)
        u[i] = d ? d[i] * x[i] : x[i];
    tqo_fwht128(u);

    for (int i = 0; i < TQO_BLOCK; ++i) {
        double t = (n == 0.0) ? 0.0 : u[i] / n;
        int c = 0;
        double dmin = INFINITY;
        for (int k = 0; k < nthr; ++k) {
            if (t >= cb->thr[k])
                ++c;
            double d = fabs(t - cb->thr[k]);
            if (d < dmin)
                dmin = d;
        }
        code[i] = c;
        if (dist)
            dist[i] = dmin;
    }
    pack_codes(cb->bits, code, field);
    *n16 = tqo_double_to_half(n > 65504.0 ? 65504.0 : n);
}

/* Decode steps: unpack, look each code up in the codebook (y_i = C[code_i]),
 * run the same transform again (v = H y) and rescale by the stored norm:
 * x_hat = (n16 / 128) * v, since H y / 128 = H^-1 y and the norm was divided
 * out before quantising.  With a diagonal d the inverse of H D is D H / 128,
 * so x_hat = d * (n16 / 128) * H y.  Result kept in double (the caller may
 * round it). */
static void decode_block(const codebook_t *cb, const uint8_t *field, uint16_t n16,
                         double *xhat, const double *d)
{
    int code[TQO_BLOCK];
    unpack_codes(cb->bits, field, code);
    for (int i = 0; i < TQO_BLOCK; ++i)
        xhat[i] = cb->levels[code[i]];
    tqo_fwht128(xhat);
    double s = tqo_half_to_double(n16) / 128.0;
    for (int i = 0; i < TQO_BLOCK; ++i)
        xhat[i] *= d ? d[i] * s : s;
}

/* ------------------------------------------------------------------------ */
/* Threading helper: split [0, n) into contiguous ranges.                   */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);
typedef struct {
    range_fn fn;
    void *ctx;
    int64_t lo, hi;
} range_job;

static void *range_thread(void *p)
{
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > n)
        nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[256];
    range_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, range_thread, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Flat block lists.                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    codebook_t cb;
    const uint16_t *x;
    uint8_t *codes;
    uint16_t *norms;
    double *dist;
    const double *d;
} enc_blocks_ctx;

static void enc_blocks_range(void *p, int64_t lo, int64_t hi)
{
    enc_blocks_ctx *c = (enc_blocks_ctx *)p;
    int cbytes = 16 * c->cb.bits;
    for (int64_t b = lo; b < hi; ++b)
        encode_block(&c->cb, c->x + b * TQO_BLOCK, c->codes + b * cbytes, c->norms + b,
                     c->dist ? c->dist + b * TQO_BLOCK : NULL, c->d);
}

int tqo_encode_blocks(int bits, const uint16_t *x, int64_t nblocks, uint8_t *codes,
                      uint16_t *norms, double *dist, const double *d, int nthreads)
{
    enc_blocks_ctx c;
    if (get_codebook(bits, &c.cb) || nblocks < 0)
        return -1;
    c.x = x;
    c.codes = codes;
    c.norms = norms;
    c.dist = dist;
    c.d = d;
    parallel_for(nblocks, nthreads, enc_blocks_range, &c);
    return 0;
}

typedef struct {
    codebook_t cb;
    const uint8_t *codes;
    const uint16_t *norms;
    double *xhat;
    uint16_t *x16;
    const double *d;
} dec_blocks_ctx;

static void dec_blocks_range(void *p, int64_t lo, int64_t hi)
{
    dec_blocks_ctx *c = (dec_blocks_ctx *)p;
    int cbytes = 16 * c->cb.bits;
    double v[TQO_BLOCK];
    for (int64_t b = lo; b < hi; ++b) {
        decode_block(&c->cb, c->codes + b * cbytes, c->norms[b], v, c->d);
        for (int i = 0; i < TQO_BLOCK; ++i) {
            if (c->xhat)
                c->xhat[b * TQO_BLOCK + i] = v[i];
            if (c->x16)
                c->x16[b * TQO_BLOCK + i] = tqo_double_to_half(v[i]);
        }
    }
}

int tqo_decode_blocks(int bits, const uint8_t *codes, const uint16_t *norms, int64_t nblocks,
                      double *xhat, uint16_t *x16, const double *d, int nthreads)
{
    dec_blocks_ctx c;
    if (get_codebook(bits, &c.cb) || nblocks < 0)
        return -1;
    c.codes = codes;
    c.norms = norms;
    c.xhat = xhat;
    c.x16 = x16;
    c.d = d;
    parallel_for(nblocks, nthreads, dec_blocks_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Tensors: x [L,H,T,D] fp16; cache codes [L,H,Tc,D/128,16*bits] u8 and     */
/* norms [L,H,Tc,D/128] fp16.  A row of D = 128*m values is m independent   */
/* blocks (head_dim 256 = two stacked 128-blocks).                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    codebook_t cb;
    const uint16_t *x;
    int64_t L, H, T, D, Tc, t0;
    uint8_t *codes;
    uint16_t *norms;
    double *dist;
    const double *d;
} enc_ctx;

/* one work item = one (l, h) pair */
static void enc_range(void *p, int64_t lo, int64_t hi)
{
    enc_ctx *c = (enc_ctx *)p;
    int64_t m = c->D / TQO_BLOCK;
    int cbytes = 16 * c->cb.bits;
    for (int64_t lh = lo; lh < hi; ++lh)
        for (int64_t t = 0; t < c->T; ++t)
            for (int64_t j = 0; j < m; ++j) {
                int64_t src = (lh * c->T + t) * m + j;          /* block of x */
                int64_t dst = (lh * c->Tc + c->t0 + t) * m + j; /* cache row t0 + t */
                encode_block(&c->cb, c->x + src * TQO_BLOCK, c->codes + dst * cbytes,
                             c->norms + dst, c->dist ? c->dist + src * TQO_BLOCK : NULL, c->d);
            }
}

int tqo_encode(int bits, const uint16_t *x, int64_t L, int64_t H, int64_t T, int64_t D,
               uint8_t *codes, uint16_t *norms, int64_t Tc, int64_t t0, double *dist,
               const double *d, int nthreads)
{
    enc_ctx c;
    if (get_codebook(bits, &c.cb) || D <= 0 || D % TQO_BLOCK || L < 0 || H < 0 || T < 0 ||
        t0 < 0 || t0 + T > Tc)
        return -1;
    c.x = x;
    c.L = L; c.H = H; c.T = T; c.D = D; c.Tc = Tc; c.t0 = t0;
    c.codes = codes;
    c.norms = norms;
    c.dist = dist;
    c.d = d;
    parallel_for(L * H, nthreads, enc_range, &c);
    return 0;
}

typedef struct {
    codebook_t cb;
    const uint8_t *codes;
    const uint16_t *norms;
    int64_t L, H, Tc, D, t0, T;
    double *xhat;
    uint16_t *x16;
    const double *d;
} dec_ctx;

static void dec_range(void *p, int64_t lo, int64_t hi)
{
    dec_ctx *c = (dec_ctx *)p;
    int64_t m = c->D / TQO_BLOCK;
    int cbytes = 16 * c->cb.bits;
    double v[TQO_BLOCK];
    for (int64_t lh = lo; lh < hi; ++lh)
        for (int64_t t = 0; t < c->T; ++t)
            for (int64_t j = 0; j < m; ++j) {
                int64_t src = (lh * c->Tc + c->t0 + t) * m + j;
                int64_t dst = (lh * c->T + t) * m + j;
                decode_block(&c->cb, c->codes + src * cbytes, c->norms[src], v, c->d);
                for (int i = 0; i < TQO_BLOCK; ++i) {
                    if (c->xhat)
                        c->xhat[dst * TQO_BLOCK + i] = v[i];
                    if (c->x16)
                        c->x16[dst * TQO_BLOCK + i] = tqo_double_to_half(v[i]);
                }
            }
}

int tqo_decode(int bits, const uint8_t *codes, const uint16_t *norms, int64_t L, int64_t H,
               int64_t Tc, int64_t D, int64_t t0, int64_t T, double *xhat, uint16_t *x16,
               const double *d, int nthreads)
{
    dec_ctx c;
    if (get_codebook(bits, &c.cb) || D <= 0 || D % TQO_BLOCK || L < 0 || H < 0 || T < 0 ||
        t0 < 0 || t0 + T > Tc)
        return -1;
    c.codes = codes;
    c.norms = norms;
    c.L = L; c.H = H; c.Tc = Tc; c.D = D; c.t0 = t0; c.T = T;
    c.xhat = xhat;
    c.x16 = x16;
    c.d = d;
    parallel_for(L * H, nthreads, dec_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Scores of queries against a compressed key cache.                        */
/* ------------------------------------------------------------------------ */

/* s[b,h,t] = scale * sum_d q[b,h,d] * k_hat[b, h / G, t, d], G = Hq / Hkv,
 * k_hat the (unrounded, double) decode of cache row t.  This is the plain
 * definition of the attention logits q.K^T * scale with grouped-query heads
 * (query heads h = g*G .. g*G+G-1 read key/value head g), over the dequantised
 * keys; nothing is rounded to FP16 on the way (the fused read path never
 * materialises FP16 keys).  One work item = one (b, kv head) pair. */
typedef struct {
    codebook_t cb;
    const uint8_t *codes;
    const uint16_t *norms;
    int64_t B, Hkv, Tc, D, T, Hq;
    const uint16_t *q;
    double scale;
    double *scores;
    const double *d;
} qk_ctx;

static void qk_range(void *p, int64_t lo, int64_t hi)
{
    qk_ctx *c = (qk_ctx *)p;
    int64_t m = c->D / TQO_BLOCK, G = c->Hq / c->Hkv;
    int cbytes = 16 * c->cb.bits;
    double *k = (double *)malloc(sizeof(double) * (size_t)c->D);
    double *qd = (double *)malloc(sizeof(double) * (size_t)(c->D * G));
    for (int64_t bg = lo; bg < hi; ++bg) {
        int64_t b = bg / c->Hkv, g = bg % c->Hkv;
        for (int64_t r = 0; r < G; ++r)
            for (int64_t d = 0; d < c->D; ++d)
                qd[r * c->D + d] = tqo_half_to_double(c->q[(b * c->Hq + g * G + r) * c->D + d]);
        for (int64_t t = 0; t < c->T; ++t) {
            for (int64_t j = 0; j < m; ++j) {
                int64_t blk = (bg * c->Tc + t) * m + j;
                decode_block(&c->cb, c->codes + blk * cbytes, c->norms[blk], k + j * TQO_BLOCK, c->d);
            }
            for (int64_t r = 0; r < G; ++r) {
                double s = 0.0;
                for (int64_t d = 0; d < c->D; ++d)
                    s += qd[r * c->D + d] * k[d];
                c->scores[(b * c->Hq + g * G + r) * c->T + t] = c->scale * s;
            }
        }
    }
    free(k);
    free(qd);
}

int tqo_qk(int bits, const uint8_t *k_codes, const uint16_t *k_norms, int64_t B, int64_t Hkv,
           int64_t Tc, int64_t D, int64_t T, const uint16_t *q, int64_t Hq, double scale,
           double *scores, const double *d, int nthreads)
{
    qk_ctx c;
    if (get_codebook(bits, &c.cb) || D <= 0 || D % TQO_BLOCK || B < 0 || Hkv <= 0 || Hq <= 0 ||
        Hq % Hkv || T < 0 || T > Tc)
        return -1;
    c.codes = k_codes;
    c.norms = k_norms;
    c.B = B; c.Hkv = Hkv; c.Tc = Tc; c.D = D; c.T = T; c.Hq = Hq;
    c.q = q;
    c.scale = scale;
    c.scores = scores;
    c.d = d;
    parallel_for(B * Hkv, nthreads, qk_range, &c);
    return 0;
}

/* Decode attention of one query token per (sequence, query head) over the
 * compressed K and V caches: out[b,h,:] = sum_t p_t * v_hat[b,h/G,t,:] with
 * p = softmax_t(scale * q[b,h,:] . k_hat[b,h/G,t,:]) over cache rows t in
 * [0, T).  The article's closing section ("現在の実装と、これから") names this
 * fusion -- attention read straight from the compressed cache -- as the next
 * step; the arithmetic is the plain definition of scaled dot-product attention
 * with grouped-query heads: max-subtracted exponentials, their sum, the weighted
 * sum of the dequantised values, all in binary64 and from the unrounded decodes.
 * One work item = one (b, kv head) pair. */
typedef struct {
    codebook_t cb;
    const uint8_t *kc, *vc;
    const uint16_t *kn, *vn;
    int64_t B, Hkv, Tc, D, T, Hq;
    const uint16_t *q;
    double scale;
    double *out;
    const double *d;
} attn_ctx;

static void attn_range(void *p, int64_t lo, int64_t hi)
{
    attn_ctx *c = (attn_ctx *)p;
    int64_t m = c->D / TQO_BLOCK, G = c->Hq / c->Hkv;
    int cbytes = 16 * c->cb.bits;
    double *row = (double *)malloc(sizeof(double) * (size_t)c->D);
    double *qd = (double *)malloc(sizeof(double) * (size_t)(c->D * G));
    double *s = (double *)malloc(sizeof(double) * (size_t)(c->T * G));
    for (int64_t bg = lo; bg < hi; ++bg) {
        int64_t b = bg / c->Hkv, g = bg % c->Hkv;
        for (int64_t r = 0; r < G; ++r)
            for (int64_t d = 0; d < c->D; ++d)
                qd[r * c->D + d] = tqo_half_to_double(c->q[(b * c->Hq + g * G + r) * c->D + d]);
        /* logits */
        for (int64_t t = 0; t < c->T; ++t) {
            for (int64_t j = 0; j < m; ++j) {
                int64_t blk = (bg * c->Tc + t) * m + j;
                decode_block(&c->cb, c->kc + blk * cbytes, c->kn[blk], row + j * TQO_BLOCK, c->d);
            }
            for (int64_t r = 0; r < G; ++r) {
                double acc = 0.0;
                for (int64_t d = 0; d < c->D; ++d)
                    acc += qd[r * c->D + d] * row[d];
                s[r * c->T + t] = c->scale * acc;
            }
        }
        /* softmax weights: exp(s - max) / sum */
        for (int64_t r = 0; r < G; ++r) {
            double mx = s[r * c->T];
            for (int64_t t = 1; t < c->T; ++t)
                if (s[r * c->T + t] > mx)
                    mx = s[r * c->T + t];
            double sum = 0.0;
            for (int64_t t = 0; t < c->T; ++t) {
                s[r * c->T + t] = exp(s[r * c->T + t] - mx);
                sum += s[r * c->T + t];
            }
            for (int64_t t = 0; t < c->T; ++t)
                s[r * c->T + t] /= sum;
        }
        /* weighted sum of the dequantised values */
        for (int64_t r = 0; r < G; ++r)
            for (int64_t d = 0; d < c->D; ++d)
                c->out[(b * c->Hq + g * G + r) * c->D + d] = 0.0;
        for (int64_t t = 0; t < c->T; ++t) {
            for (int64_t j = 0; j < m; ++j) {
                int64_t blk = (bg * c->Tc + t) * m + j;
                decode_block(&c->cb, c->vc + blk * cbytes, c->vn[blk], row + j * TQO_BLOCK, c->d);
            }
            for (int64_t r = 0; r < G; ++r) {
                double w = s[r * c->T + t];
                double *o = c->out + (b * c->Hq + g * G + r) * c->D;
                for (int64_t d = 0; d < c->D; ++d)
                    o[d] += w * row[d];
            }
        }
    }
    free(row);
    free(qd);
    free(s);
}

int tqo_attn_decode(int bits, const uint8_t *k_codes, const uint16_t *k_norms,
                    const uint8_t *v_codes, const uint16_t *v_norms, int64_t B, int64_t Hkv,
                    int64_t Tc, int64_t D, int64_t T, const uint16_t *q, int64_t Hq, double scale,
                    double *out, const double *d, int nthreads)
{
    attn_ctx c;
    if (get_codebook(bits, &c.cb) || D <= 0 || D % TQO_BLOCK || B < 0 || Hkv <= 0 || Hq <= 0 ||
        Hq % Hkv || T < 1 || T > Tc)
        return -1;
    c.kc = k_codes;
    c.kn = k_norms;
    c.vc = v_codes;
    c.vn = v_norms;
    c.B = B; c.Hkv = Hkv; c.Tc = Tc; c.D = D; c.T = T; c.Hq = Hq;
    c.q = q;
    c.scale = scale;
    c.out = out;
    c.d = d;
    parallel_for(B * Hkv, nthreads, attn_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Interleaved block records.                                               */
/* ------------------------------------------------------------------------ */

/* Section "どこまで小さくなるのか": each block packs its 128 values and one FP16
 * norm (50 / 34 bytes).  Record layout (this oracle's reading; the page fixes
 * only the content and the size): the norm's two bytes, little-endian, then
 * the block's 16*bits code bytes; records in block order.  Byte copies only. */
int tqo_pack_records(int bits, const uint8_t *codes, const uint16_t *norms, int64_t nblocks,
                     uint8_t *records)
{
    if ((bits != 2 && bits != 3) || nblocks < 0)
        return -1;
    int cb = 16 * bits, rb = cb + 2;
    for (int64_t b = 0; b < nblocks; ++b) {
        uint8_t *r = records + b * rb;
        r[0] = (uint8_t)(norms[b] & 0xFF);
        r[1] = (uint8_t)(norms[b] >> 8);
        for (int i = 0; i < cb; ++i)
            r[2 + i] = codes[b * cb + i];
    }
    return 0;
}

int tqo_unpack_records(int bits, const uint8_t *records, int64_t nblocks, uint8_t *codes,
                       uint16_t *norms)
{
    if ((bits != 2 && bits != 3) || nblocks < 0)
        return -1;
    int cb = 16 * bits, rb = cb + 2;
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *r = records + b * rb;
        norms[b] = (uint16_t)(r[0] | (r[1] << 8));
        for (int i = 0; i < cb; ++i)
            codes[b * cb + i] = r[2 + i];
    }
    return 0;
}
