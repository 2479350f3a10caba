/*
 * tq_oracle.h -- declarations of the CPU oracle of the turbo3 / turbo2 block
 * codec.  TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline);
 * the product library never includes this header and this header includes
 * nothing of the product's.
 *
 * All floating point is binary64.  fp16 values travel as their uint16 bit
 * patterns.  Functions that take nthreads split independent blocks / rows
 * over that many POSIX threads.  Every int-returning function returns 0 on
 * success and -1 on invalid arguments (codebook solvers return the number of
 * iterations instead).
 *
 * d (optional, NULL for none): 128 signs +-1.0 of the randomised rotation H D
 * (encode rotates H (d * x); decode returns d * (n16 / 128) H y).  Every block
 * of a call uses the same d.
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H

#include <stdint.h>

#define TQO_BLOCK 128

#ifdef __cplusplus
extern "C" {
#endif

double tqo_half_to_double(uint16_t h);
uint16_t tqo_double_to_half(double x);

/* N(0,1) Lloyd-Max codebook with 2^bits ascending levels and 2^bits-1
 * thresholds, bits in 1..4.  Returns iterations used, -1 on failure. */
int tqo_codebook(int bits, double *levels, double *thresholds);

/* In place, unnormalised Sylvester-Hadamard transform of 128 values. */
void tqo_fwht128(double *v);

/* Contiguous lists of blocks: x is nblocks*128 fp16, codes nblocks*16*bits
 * bytes, norms nblocks fp16, dist (optional) nblocks*128 doubles. */
int tqo_encode_blocks(int bits, const uint16_t *x, int64_t nblocks, uint8_t *codes,
                      uint16_t *norms, double *dist, const double *d, int nthreads);
/* xhat (optional) nblocks*128 doubles; x16 (optional) the same rounded to fp16. */
int tqo_decode_blocks(int bits, const uint8_t *codes, const uint16_t *norms, int64_t nblocks,
                      double *xhat, uint16_t *x16, const double *d, int nthreads);

/* Tensor forms: x [L,H,T,D]; cache codes [L,H,Tc,D/128,16*bits], norms
 * [L,H,Tc,D/128]; encode writes cache rows [t0, t0+T), decode reads them. */
int tqo_encode(int bits, const uint16_t *x, int64_t L, int64_t H, int64_t T, int64_t D,
               uint8_t *codes, uint16_t *norms, int64_t Tc, int64_t t0, double *dist,
               const double *d, int nthreads);
int tqo_decode(int bits, const uint8_t *codes, const uint16_t *norms, int64_t L, int64_t H,
               int64_t Tc, int64_t D, int64_t t0, int64_t T, double *xhat, uint16_t *x16,
               const double *d, int nthreads);

/* Key cache [B,Hkv,Tc,D/128] packed, q fp16 [B,Hq,D], scores [B,Hq,T] (double)
 * over cache rows [0, T). */
int tqo_qk(int bits, const uint8_t *k_codes, const uint16_t *k_norms, int64_t B, int64_t Hkv,
           int64_t Tc, int64_t D, int64_t T, const uint16_t *q, int64_t Hq, double scale,
           double *scores, const double *d, int nthreads);

/* Decode attention: K and V caches [B,Hkv,Tc,D/128] packed, q fp16 [B,Hq,D],
 * out [B,Hq,D] (double) = softmax over rows [0, T) of scale * q.k_hat, applied
 * to v_hat.  T >= 1. */
int tqo_attn_decode(int bits, const uint8_t *k_codes, const uint16_t *k_norms,
                    const uint8_t *v_codes, const uint16_t *v_norms, int64_t B, int64_t Hkv,
                    int64_t Tc, int64_t D, int64_t T, const uint16_t *q, int64_t Hq, double scale,
                    double *out, const double *d, int nthreads);

/* Interleaved records of 2 + 16*bits bytes per block (the fp16 norm, little-
 * endian, then the code bytes) from / to the two planes. */
int tqo_pack_records(int bits, const uint8_t *codes, const uint16_t *norms, int64_t nblocks,
                     uint8_t *records);
int tqo_unpack_records(int bits, const uint8_t *records, int64_t nblocks, uint8_t *codes,
                       uint16_t *norms);

#ifdef __cplusplus
}
#endif
#endif
