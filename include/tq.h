/*
 * tq.h -- C ABI of the turbo3 / turbo2 KV-cache block codec for AMD MI355X
 * (gfx950).  Plain C: no C++ types, no exceptions and no torch types cross
 * this boundary.
 *
 * The method is the one described in "llama.cpp に TurboQuant を実装 -- 2bit・
 * 3bit の KV キャッシュ圧縮" (openalchemy.io):
 *   - section "TurboQuant の何が違うのか": rotate before quantising, with a fast
 *     Walsh-Hadamard transform (additions and subtractions only, self-inverse)
 *     in place of a dense random rotation, then an optimal per-coordinate
 *     Lloyd-Max scalar quantiser; the rotation is undone on read;
 *   - section "どこまで小さくなるのか": a block is 128 values plus one FP16
 *     norm (50 bytes for turbo3, 34 bytes for turbo2);
 *   - section "実モデルでの数値": a head_dim of 128*m is m stacked blocks;
 *   - section "現在の実装と、これから": the cache is stored compressed and
 *     dequantised before attention today (tq_decode); the next step fuses the
 *     dequantisation into the attention tiles so keys never exist in FP16
 *     (tq_qk_scores).
 *
 * Block format (the page fixes only the byte counts; this layout is this
 * library's convention):
 *   - for a fp16 tensor [L, H, T, D] with D = 128*m, row (l, h, t) holds the m
 *     blocks (l, h, t, j), j = 0..m-1, each 128 consecutive values;
 *   - per block:  n = ||x||_2;  u = H x (unnormalised Sylvester-Hadamard
 *     matrix, natural order, H H = 128 I);  t = u / n;
 *     code_i = #{k : t_i >= tau_k}, tau the N(0,1) Lloyd-Max thresholds
 *     (7 for turbo3, 3 for turbo2; a value on a threshold takes the upper
 *     cell); a zero block gets every code = 2^bits / 2 and n = 0;
 *   - decode: x_hat = (n16 / 128) * H * C[code], C the Lloyd-Max levels;
 *   - a cache is two planes: codes u8 [L, H, Tc, m, 16*bits] (128 codes as one
 *     little-endian bit stream, code i at bits [bits*i, bits*i + bits)) and
 *     norms fp16 [L, H, Tc, m] (round to nearest even, saturating at 65504).
 *     16*bits + 2 bytes per block: 50 (0.39 B/value) and 34 (0.27 B/value).
 *
 * Memory and streams: every pointer named "device" is device memory the
 * caller owns (e.g. from torch on ROCm).  The library allocates, frees and
 * synchronises nothing and keeps no per-call state (the exceptions are the
 * per-thread timing hook, tq_time_next_launch, and the static device scratch array
 * that tq_attn_decode_noalloc uses instead of a workspace).  stream is a hipStream_t
 * passed as void* (NULL = the default stream); calls are asynchronous on it
 * and their results are valid once the caller has synchronised that stream.
 *
 * Environment (read once per process, tuning only): TQ_ENCODE_GROUPS_PER_CU,
 * TQ_ENCODE_ROT_GROUPS_PER_CU and TQ_DECODE_GROUPS_PER_CU cap the workgroups
 * per compute unit of the encode / randomised-rotation encode / decode grids
 * (0 = no cap; defaults 0, 2 and 0).  Every block is coded independently, so
 * results are the same for every value; only the launch shape changes.
 *
 * Errors: arguments are checked on the host before any HIP call; a failed
 * check returns a negative tq_status and launches nothing.  Work of size zero
 * returns TQ_OK and launches nothing.  A launch that HIP reports as failed
 * returns TQ_ERR_DEVICE.  Non-finite inputs are outside the contract: they do
 * not fault, but their outputs are unspecified.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache types; the value is the number of bits per code. */
enum tq_type { TQ_TURBO2 = 2, TQ_TURBO3 = 3 };

enum tq_status {
    TQ_OK = 0,
    TQ_ERR_TYPE = -1,   /* type is not TQ_TURBO2 / TQ_TURBO3 */
    TQ_ERR_SHAPE = -2,  /* negative size, D not a positive multiple of 128, Hq % Hkv, limits */
    TQ_ERR_RANGE = -3,  /* t0 < 0 or t0 + T > Tc */
    TQ_ERR_NULL = -4,   /* NULL pointer where there is work to do */
    TQ_ERR_ALIGN = -5,  /* x / q / codes not 16-byte, norms not 2-byte, scores not 4-byte aligned */
    TQ_ERR_ALIAS = -6,  /* an output range overlaps an input range or another output */
    TQ_ERR_DEVICE = -7,      /* HIP reported an error for the launch */
    TQ_ERR_WORKSPACE = -8    /* workspace smaller than tq_attn_workspace_bytes */
};

/* Largest head_dim tq_qk_scores accepts (16 blocks per vector). */
#define TQ_QK_MAX_D 2048

/* Bytes of packed codes per block: 48 (turbo3), 32 (turbo2); TQ_ERR_TYPE otherwise. */
int tq_block_code_bytes(int type);
/* Bytes per block including its fp16 norm: 50 (turbo3), 34 (turbo2); TQ_ERR_TYPE otherwise. */
int tq_block_bytes(int type);
/* Size of the codes plane of a [L, H, Tc, D] cache in bytes; negative tq_status on bad input. */
int64_t tq_codes_nbytes(int type, int64_t L, int64_t H, int64_t Tc, int64_t D);
/* Number of fp16 norms of a [L, H, Tc, D] cache; negative tq_status on bad input. */
int64_t tq_norms_count(int64_t L, int64_t H, int64_t Tc, int64_t D);
/* Static string naming a status code (never NULL). */
const char *tq_status_string(int status);

/* The float32 codebook the kernels use (host memory, computed by this library
 * from the N(0,1) Lloyd-Max conditions): levels[2^type] ascending,
 * thresholds[2^type - 1] (midpoints of adjacent levels).  Section
 * "TurboQuant の何が違うのか" asks for the optimal Lloyd-Max codebook; the
 * Gaussian is this library's reading.  Returns TQ_OK or TQ_ERR_TYPE/TQ_ERR_NULL. */
int tq_codebook(int type, float *levels, float *thresholds);

/* Encode (the cache write path: rotate + quantise + pack, section
 * "TurboQuant の何が違うのか"; T = 1 is the per-token append of a decode step).
 *   x      device fp16 [L, H, T, D], contiguous, 16-byte aligned (read only)
 *   codes  device u8 [L, H, Tc, D/128, 16*type], 16-byte aligned
 *   norms  device fp16 [L, H, Tc, D/128], 2-byte aligned
 * Writes cache rows [t0, t0 + T) of every (l, h); other rows are untouched.
 * Requires D % 128 == 0, 0 <= t0, t0 + T <= Tc, fewer than 2^31 blocks. */
int tq_encode(int type, const void *x, int64_t L, int64_t H, int64_t T, int64_t D,
              void *codes, void *norms, int64_t Tc, int64_t t0, void *stream);

/* Decode (dequantise to fp16 before attention, section "現在の実装と、これから"):
 *   codes, norms  device cache planes of a [L, H, Tc, D] cache (read only)
 *   x             device fp16 [L, H, T, D], contiguous, 16-byte aligned
 * Reads cache rows [t0, t0 + T) and writes x_hat rounded to fp16 (nearest even). */
int tq_decode(int type, const void *codes, const void *norms, int64_t L, int64_t H,
              int64_t Tc, int64_t D, int64_t t0, int64_t T, void *x, void *stream);

/* Fused read of a compressed key cache (the fusion named in section
 * "現在の実装と、これから": keys are never materialised in fp16):
 *   k_codes, k_norms  device key cache of shape [B, Hkv, Tc, D] (read only)
 *   q                 device fp16 [B, Hq, D], 16-byte aligned (read only)
 *   scores            device fp32 [B, Hq, T], 4-byte aligned
 * scores[b, h, t] = scale * sum_d q[b, h, d] * k_hat[b, h / G, t, d] for cache
 * rows t in [0, T), G = Hq / Hkv (query heads h = g*G .. g*G + G - 1 share key
 * head g), k_hat the decoded key kept in float (not rounded to fp16).
 * Requires Hq % Hkv == 0, T <= Tc, D % 128 == 0 and D <= TQ_QK_MAX_D. */
int tq_qk_scores(int type, const void *k_codes, const void *k_norms, int64_t B, int64_t Hkv,
                 int64_t Tc, int64_t D, int64_t T, const void *q, int64_t Hq, float scale,
                 float *scores, void *stream);

/* Bytes of device workspace tq_attn_decode needs for these sizes (0 when B == 0);
 * a negative tq_status for sizes tq_attn_decode would reject.  Depends on the sizes
 * only, not on the device. */
int64_t tq_attn_workspace_bytes(int type, int64_t B, int64_t Hkv, int64_t Tc, int64_t D,
                                int64_t T, int64_t Hq);

/* Decode attention straight from the compressed caches: the fused read of section
 * "現在の実装と、これから" carried through softmax and the values, one query
 * token per (sequence, query head):
 *   k_codes, k_norms, v_codes, v_norms  device K and V caches [B, Hkv, Tc, D] (read only)
 *   q          device fp16 [B, Hq, D], 16-byte aligned (read only)
 *   out        device fp32 [B, Hq, D], 4-byte aligned
 *   workspace  device, at least tq_attn_workspace_bytes(...) bytes, 16-byte aligned;
 *              scratch for per-chunk partial results, overwritten, no initial
 *              contents needed; calls that share a workspace must not overlap
 * out[b, h, :] = sum_t p_t v_hat[b, h/G, t, :] with p = softmax over rows t in [0, T)
 * of scale * q[b, h, :] . k_hat[b, h/G, t, :], G = Hq / Hkv, k_hat and v_hat the
 * decoded keys and values kept in float.  D is 128 or 256 (section "実モデルでの数値":
 * a head_dim of 256 is two stacked blocks, each with its own norm; a row's score sums
 * both blocks' dot products).  Requires T >= 1 (when B > 0), T <= Tc,
 * T <= 65535 * 1024, Hq % Hkv == 0, B * Hkv * Tc * D / 128 <= 2^40 and
 * B * Hq <= 2^29 - 1; other sizes return TQ_ERR_SHAPE.  Two kernel launches on
 * `stream`. */
int tq_attn_decode(int type, const void *k_codes, const void *k_norms, const void *v_codes,
                   const void *v_norms, int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T,
                   const void *q, int64_t Hq, float scale, float *out, void *workspace,
                   int64_t workspace_bytes, void *stream);

/* Interleaved block records (each block packs its 128 values and one FP16 norm,
 * section "どこまで小さくなるのか": 50 B turbo3, 34 B turbo2), the llama.cpp-style
 * block struct { fp16 norm (little-endian); uint8 codes[16*type]; }, records in block
 * order, for interchange with code that expects one record per block:
 *   codes    device codes plane of nblocks blocks (16*type bytes each), 16-byte aligned
 *   norms    device norms plane of nblocks fp16 values, 2-byte aligned
 *   records  device nblocks * (2 + 16*type) bytes, 16-byte aligned
 * Block b of the planes <-> record b.  A sub-range of a cache is converted by passing
 * pointers offset to its first block (records then stay 16-byte aligned for block
 * offsets that are multiples of 8).  Requires 0 <= nblocks < 2^31.  Byte moves only:
 * a pack followed by an unpack restores both planes exactly. */
int tq_pack_records(int type, const void *codes, const void *norms, int64_t nblocks,
                    void *records, void *stream);
int tq_unpack_records(int type, const void *records, int64_t nblocks, void *codes, void *norms,
                      void *stream);

/* Randomised rotation.  TurboQuant rotates each vector by a random orthogonal matrix
 * before quantising (section "TurboQuant の何が違うのか"); the calls above use the
 * fixed Hadamard H.  The _rot variants below use H D instead, D a diagonal of signs:
 *   signs  host memory, 4 words (128 bits), or NULL (then exactly the call above);
 *          bit p % 32 of signs[p / 32] set <=> D_pp = -1, for value position p of
 *          every 128-value block.  Read during the call only.
 * Encode rotates u = H D x; decode returns D (n16/128) H y; q.K and the attention
 * decode the keys and values the same way (internally q' = H D q and a final D on
 * the attention output).  A cache written with some signs must be read with the same
 * signs.  The signs are an input: callers draw them (for instance from a seed) and
 * keep them with the cache.  Otherwise each _rot call takes the arguments, has the
 * layouts and returns the statuses of the call it extends.
 * Effect: an input aligned with a row of H, which H alone collapses onto a single
 * coordinate, is spread over all coordinates; a one-hot input stays flat under any
 * H D (its round trip is the same as without signs). */
int tq_encode_rot(int type, const uint32_t *signs, const void *x, int64_t L, int64_t H,
                  int64_t T, int64_t D, void *codes, void *norms, int64_t Tc, int64_t t0,
                  void *stream);
int tq_decode_rot(int type, const uint32_t *signs, const void *codes, const void *norms,
                  int64_t L, int64_t H, int64_t Tc, int64_t D, int64_t t0, int64_t T, void *x,
                  void *stream);
int tq_qk_scores_rot(int type, const uint32_t *signs, const void *k_codes, const void *k_norms,
                     int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T, const void *q,
                     int64_t Hq, float scale, float *scores, void *stream);
int tq_attn_decode_rot(int type, const uint32_t *signs, const void *k_codes,
                       const void *k_norms, const void *v_codes, const void *v_norms, int64_t B,
                       int64_t Hkv, int64_t Tc, int64_t D, int64_t T, const void *q, int64_t Hq,
                       float scale, float *out, void *workspace, int64_t workspace_bytes,
                       void *stream);

/* Decode attention that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The call of tq_attn_decode_rot (signs: as
 * there, NULL = plain H) with the workspace taken from a static device array of
 * TQ_ATTN_SCRATCH_BYTES inside the library: one copy per device the library runs on,
 * held until the process ends, its address looked up once per device on the first
 * call there.  Same arguments (less workspace and workspace_bytes), layouts, results
 * and statuses; in addition TQ_ERR_WORKSPACE when the sizes need more than
 * TQ_ATTN_SCRATCH_BYTES (tq_attn_workspace_bytes(...) > TQ_ATTN_SCRATCH_BYTES: about
 * 15,000 (sequence, query head, row chunk) partials; the decode step of 16 sequences x
 * 32 heads at 32768 rows needs 2.2 MB), and TQ_ERR_DEVICE when the array's address
 * cannot be found.  No hipMalloc, hipFree or memset.  Every call on a device uses that
 * device's one array: calls that overlap on the same device (other streams, other
 * threads) race on it and must be serialised by the caller.  The array needs no initial
 * contents (every partial is written before it is read). */
#define TQ_ATTN_SCRATCH_BYTES (8 << 20)
int tq_attn_decode_noalloc(int type, const uint32_t *signs, const void *k_codes,
                           const void *k_norms, const void *v_codes, const void *v_norms,
                           int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T,
                           const void *q, int64_t Hq, float scale, float *out, void *stream);

/* Timing hook: a measurement aid, not an operation of the codec.
 * The next kernel this thread launches through any tq_* call records its own start
 * and stop on these events.  The timestamps are those of the kernel's dispatch
 * packet (hipExtLaunchKernelGGL), as a kernel trace reports them, without the
 * dispatch latency that events recorded around the call add.  The hook then clears
 * itself.
 * start_event, stop_event: hipEvent_t created by the caller with timing enabled,
 *   passed as void*; either may be NULL (that side is not recorded); both NULL
 *   clears a pending hook.
 * A call that launches two kernels (tq_attn_decode) times the first; a call that
 * returns an error before launching leaves the hook pending.  Per thread; the
 * library never waits on the events.  Returns TQ_OK. */
int tq_time_next_launch(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
