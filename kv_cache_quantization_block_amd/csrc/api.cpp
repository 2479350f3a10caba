// api.cpp -- the extern "C" entry points of libtq: argument checks on the host,
// then one asynchronous kernel launch on the caller's stream.  No allocation,
// no synchronisation, no state beyond the process-wide constant codebooks.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include "internal.h"
#include "tq.h"

namespace {

bool valid_type(int type) { return type == TQ_TURBO2 || type == TQ_TURBO3; }

// a * b into *out, false on int64 overflow or negative operands
bool mul(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0)
        return false;
    return !__builtin_mul_overflow(a, b, out);
}

bool mul4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t *out)
{
    int64_t ab, abc;
    return mul(a, b, &ab) && mul(ab, c, &abc) && mul(abc, d, out);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The caller's four sign words (host memory), or none.
tq::Signs to_signs(const uint32_t *signs)
{
    tq::Signs sg = {{0u, 0u, 0u, 0u}};
    if (signs)
        for (int k = 0; k < 4; ++k)
            sg.w[k] = signs[k];
    return sg;
}

// half-open byte ranges [p, p + n) overlap (empty ranges never do)
bool overlap(const void *p, int64_t n, const void *q, int64_t m)
{
    if (n <= 0 || m <= 0)
        return false;
    uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// Shapes shared by encode / decode: sizes non-negative, D a positive multiple
// of 128, cache rows in range, totals representable; fills the block counts.
int check_codec_shape(int type, int64_t L, int64_t H, int64_t T, int64_t D, int64_t Tc,
                      int64_t t0, int64_t *nblocks, int64_t *cache_blocks)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (L < 0 || H < 0 || T < 0 || Tc < 0 || D <= 0 || D % tq::kBlock)
        return TQ_ERR_SHAPE;
    if (t0 < 0 || T > Tc || t0 > Tc - T)
        return TQ_ERR_RANGE;
    const int64_t m = D / tq::kBlock;
    if (!mul4(L, H, T, m, nblocks) || !mul4(L, H, Tc, m, cache_blocks))
        return TQ_ERR_SHAPE;
    int64_t bytes;
    if (!mul(*cache_blocks, 256, &bytes) || *nblocks > INT32_MAX || T * m > INT32_MAX)
        return TQ_ERR_SHAPE;
    return TQ_OK;
}

}  // namespace

extern "C" {

int tq_block_code_bytes(int type) { return valid_type(type) ? 16 * type : TQ_ERR_TYPE; }

int tq_block_bytes(int type) { return valid_type(type) ? 16 * type + 2 : TQ_ERR_TYPE; }

int64_t tq_codes_nbytes(int type, int64_t L, int64_t H, int64_t Tc, int64_t D)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    int64_t blocks, bytes;
    if (D <= 0 || D % tq::kBlock || !mul4(L, H, Tc, D / tq::kBlock, &blocks) ||
        !mul(blocks, 16 * type, &bytes))
        return TQ_ERR_SHAPE;
    return bytes;
}

int64_t tq_norms_count(int64_t L, int64_t H, int64_t Tc, int64_t D)
{
    int64_t blocks;
    if (D <= 0 || D % tq::kBlock || !mul4(L, H, Tc, D / tq::kBlock, &blocks))
        return TQ_ERR_SHAPE;
    return blocks;
}

const char *tq_status_string(int status)
{
    switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_TYPE: return "TQ_ERR_TYPE: type must be TQ_TURBO2 (2) or TQ_TURBO3 (3)";
    case TQ_ERR_SHAPE: return "TQ_ERR_SHAPE: invalid or unsupported sizes";
    case TQ_ERR_RANGE: return "TQ_ERR_RANGE: cache rows [t0, t0+T) outside [0, Tc)";
    case TQ_ERR_NULL: return "TQ_ERR_NULL: null pointer";
    case TQ_ERR_ALIGN: return "TQ_ERR_ALIGN: misaligned pointer";
    case TQ_ERR_ALIAS: return "TQ_ERR_ALIAS: output overlaps another buffer";
    case TQ_ERR_DEVICE: return "TQ_ERR_DEVICE: HIP launch failed";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE: workspace smaller than tq_attn_workspace_bytes";
    default: return "unknown tq_status";
    }
}

int tq_codebook(int type, float *levels, float *thresholds)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (!levels || !thresholds)
        return TQ_ERR_NULL;
    const tq::Codebook *cb = tq::codebook(type);
    memcpy(levels, cb->levels, sizeof(float) * (1u << type));
    memcpy(thresholds, cb->thresholds, sizeof(float) * ((1u << type) - 1));
    return TQ_OK;
}

int tq_encode_rot(int type, const uint32_t *signs, const void *x, int64_t L, int64_t H,
                  int64_t T, int64_t D, void *codes, void *norms, int64_t Tc, int64_t t0,
                  void *stream)
{
    int64_t nblocks, cache_blocks;
    int rc = check_codec_shape(type, L, H, T, D, Tc, t0, &nblocks, &cache_blocks);
    if (rc != TQ_OK)
        return rc;
    if (nblocks == 0)
        return TQ_OK;
    if (!x || !codes || !norms)
        return TQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(norms, 2))
        return TQ_ERR_ALIGN;
    const int64_t xb = nblocks * 256, cb = cache_blocks * 16 * type, nbytes = cache_blocks * 2;
    if (overlap(x, xb, codes, cb) || overlap(x, xb, norms, nbytes) ||
        overlap(codes, cb, norms, nbytes))
        return TQ_ERR_ALIAS;
    const int64_t m = D / tq::kBlock;
    return tq::launch_encode(type, to_signs(signs), x, nblocks, T * m, Tc * m, t0 * m, codes,
                             norms, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}

int tq_encode(int type, const void *x, int64_t L, int64_t H, int64_t T, int64_t D, void *codes,
              void *norms, int64_t Tc, int64_t t0, void *stream)
{
    return tq_encode_rot(type, nullptr, x, L, H, T, D, codes, norms, Tc, t0, stream);
}

int tq_decode_rot(int type, const uint32_t *signs, const void *codes, const void *norms,
                  int64_t L, int64_t H, int64_t Tc, int64_t D, int64_t t0, int64_t T, void *x,
                  void *stream)
{
    int64_t nblocks, cache_blocks;
    int rc = check_codec_shape(type, L, H, T, D, Tc, t0, &nblocks, &cache_blocks);
    if (rc != TQ_OK)
        return rc;
    if (nblocks == 0)
        return TQ_OK;
    if (!x || !codes || !norms)
        return TQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(norms, 2))
        return TQ_ERR_ALIGN;
    const int64_t xb = nblocks * 256, cb = cache_blocks * 16 * type, nbytes = cache_blocks * 2;
    if (overlap(x, xb, codes, cb) || overlap(x, xb, norms, nbytes))
        return TQ_ERR_ALIAS;
    const int64_t m = D / tq::kBlock;
    return tq::launch_decode(type, to_signs(signs), codes, norms, nblocks, T * m, Tc * m, t0 * m,
                             x, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}

int tq_decode(int type, const void *codes, const void *norms, int64_t L, int64_t H, int64_t Tc,
              int64_t D, int64_t t0, int64_t T, void *x, void *stream)
{
    return tq_decode_rot(type, nullptr, codes, norms, L, H, Tc, D, t0, T, x, stream);
}

int tq_qk_scores_rot(int type, const uint32_t *signs, const void *k_codes, const void *k_norms,
                     int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T, const void *q,
                     int64_t Hq, float scale, float *scores, void *stream)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (B < 0 || Hkv <= 0 || Hq <= 0 || Tc < 0 || T < 0 || D <= 0 || D % tq::kBlock ||
        D > TQ_QK_MAX_D || Hq % Hkv)
        return TQ_ERR_SHAPE;
    if (T > Tc)
        return TQ_ERR_RANGE;
    const int64_t m = D / tq::kBlock;
    int64_t cache_blocks, nscores, qn;
    if (!mul4(B, Hkv, Tc, m, &cache_blocks) || !mul4(B, Hq, T, 1, &nscores) ||
        !mul4(B, Hq, D, 1, &qn) || cache_blocks > ((int64_t)1 << 40) ||
        T > 65535LL * 1024 || B * Hq > INT32_MAX)
        return TQ_ERR_SHAPE;
    if (B == 0 || T == 0)
        return TQ_OK;
    if (!k_codes || !k_norms || !q || !scores)
        return TQ_ERR_NULL;
    if (!aligned(k_codes, 16) || !aligned(q, 16) || !aligned(k_norms, 2) || !aligned(scores, 4))
        return TQ_ERR_ALIGN;
    const int64_t sb = nscores * 4;
    if (overlap(scores, sb, k_codes, cache_blocks * 16 * type) ||
        overlap(scores, sb, k_norms, cache_blocks * 2) || overlap(scores, sb, q, qn * 2))
        return TQ_ERR_ALIAS;
    return tq::launch_qk(type, to_signs(signs), k_codes, k_norms, B, Hkv, Tc, m, T, q, Hq, scale,
                         scores, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}

int tq_qk_scores(int type, const void *k_codes, const void *k_norms, int64_t B, int64_t Hkv,
                 int64_t Tc, int64_t D, int64_t T, const void *q, int64_t Hq, float scale,
                 float *scores, void *stream)
{
    return tq_qk_scores_rot(type, nullptr, k_codes, k_norms, B, Hkv, Tc, D, T, q, Hq, scale,
                            scores, stream);
}

int tq_pack_records(int type, const void *codes, const void *norms, int64_t nblocks,
                    void *records, void *stream)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (nblocks < 0 || nblocks > INT32_MAX)
        return TQ_ERR_SHAPE;
    if (nblocks == 0)
        return TQ_OK;
    if (!codes || !norms || !records)
        return TQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(norms, 2) || !aligned(records, 16))
        return TQ_ERR_ALIGN;
    const int64_t cb = nblocks * 16 * type, nbytes = nblocks * 2, rb = nblocks * (2 + 16 * type);
    if (overlap(records, rb, codes, cb) || overlap(records, rb, norms, nbytes))
        return TQ_ERR_ALIAS;
    return tq::launch_pack_records(type, codes, norms, nblocks, records, stream) ? TQ_ERR_DEVICE
                                                                                : TQ_OK;
}

int tq_unpack_records(int type, const void *records, int64_t nblocks, void *codes, void *norms,
                      void *stream)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (nblocks < 0 || nblocks > INT32_MAX)
        return TQ_ERR_SHAPE;
    if (nblocks == 0)
        return TQ_OK;
    if (!codes || !norms || !records)
        return TQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(norms, 2) || !aligned(records, 16))
        return TQ_ERR_ALIGN;
    const int64_t cb = nblocks * 16 * type, nbytes = nblocks * 2, rb = nblocks * (2 + 16 * type);
    if (overlap(records, rb, codes, cb) || overlap(records, rb, norms, nbytes) ||
        overlap(codes, cb, norms, nbytes))
        return TQ_ERR_ALIAS;
    return tq::launch_unpack_records(type, records, nblocks, codes, norms, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}

int tq_time_next_launch(void *start_event, void *stop_event)
{
    tq::set_next_launch_events(start_event, stop_event);
    return TQ_OK;
}

}  // extern "C"

// Shapes of the decode attention call (D = 128 or 256); fills the cache blocks of one cache.
static int check_attn_shape(int type, int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T,
                            int64_t Hq, int64_t *cache_blocks)
{
    if (!valid_type(type))
        return TQ_ERR_TYPE;
    if (B < 0 || Hkv <= 0 || Hq <= 0 || Tc < 0 || T < 0 ||
        (D != tq::kBlock && D != 2 * tq::kBlock) || Hq % Hkv || (B > 0 && T < 1))
        return TQ_ERR_SHAPE;
    if (T > Tc)
        return TQ_ERR_RANGE;
    int64_t nq;
    if (!mul4(B, Hkv, Tc, D / tq::kBlock, cache_blocks) || *cache_blocks > ((int64_t)1 << 40) ||
        !mul4(B, Hq, D, 1, &nq) || T > 65535LL * 1024 || B * Hq > INT32_MAX / 4)
        return TQ_ERR_SHAPE;
    return TQ_OK;
}

int64_t tq_attn_workspace_bytes(int type, int64_t B, int64_t Hkv, int64_t Tc, int64_t D,
                                int64_t T, int64_t Hq)
{
    int64_t cache_blocks;
    const int st = check_attn_shape(type, B, Hkv, Tc, D, T, Hq, &cache_blocks);
    if (st != TQ_OK)
        return st;
    if (B == 0)
        return 0;
    return tq::attn_workspace_bytes(type, B, Hkv, T, Hq, D / tq::kBlock);
}

int tq_attn_decode_rot(int type, const uint32_t *signs, const void *k_codes,
                       const void *k_norms, const void *v_codes, const void *v_norms, int64_t B,
                       int64_t Hkv, int64_t Tc, int64_t D, int64_t T, const void *q, int64_t Hq,
                       float scale, float *out, void *workspace, int64_t workspace_bytes,
                       void *stream)
{
    int64_t cache_blocks;
    const int st = check_attn_shape(type, B, Hkv, Tc, D, T, Hq, &cache_blocks);
    if (st != TQ_OK)
        return st;
    if (B == 0)
        return TQ_OK;
    if (!k_codes || !k_norms || !v_codes || !v_norms || !q || !out || !workspace)
        return TQ_ERR_NULL;
    if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q, 16) ||
        !aligned(k_norms, 2) || !aligned(v_norms, 2) || !aligned(out, 4) ||
        !aligned(workspace, 16))
        return TQ_ERR_ALIGN;
    const int64_t need = tq::attn_workspace_bytes(type, B, Hkv, T, Hq, D / tq::kBlock);
    if (workspace_bytes < need)
        return TQ_ERR_WORKSPACE;
    const int64_t ob = B * Hq * D * 4, cb = cache_blocks * 16 * type, nb = cache_blocks * 2;
    const void *ins[5] = {k_codes, k_norms, v_codes, v_norms, q};
    const int64_t inb[5] = {cb, nb, cb, nb, B * Hq * D * 2};
    for (int i = 0; i < 5; ++i)
        if (overlap(out, ob, ins[i], inb[i]) || overlap(workspace, need, ins[i], inb[i]))
            return TQ_ERR_ALIAS;
    if (overlap(out, ob, workspace, need))
        return TQ_ERR_ALIAS;
    return tq::launch_attn(type, to_signs(signs), k_codes, k_norms, v_codes, v_norms, B, Hkv, Tc,
                           D / tq::kBlock, T, q, Hq, scale, out, workspace, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}

int tq_attn_decode(int type, const void *k_codes, const void *k_norms, const void *v_codes,
                   const void *v_norms, int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T,
                   const void *q, int64_t Hq, float scale, float *out, void *workspace,
                   int64_t workspace_bytes, void *stream)
{
    return tq_attn_decode_rot(type, nullptr, k_codes, k_norms, v_codes, v_norms, B, Hkv, Tc, D, T,
                              q, Hq, scale, out, workspace, workspace_bytes, stream);
}

int tq_attn_decode_noalloc(int type, const uint32_t *signs, const void *k_codes,
                           const void *k_norms, const void *v_codes, const void *v_norms,
                           int64_t B, int64_t Hkv, int64_t Tc, int64_t D, int64_t T,
                           const void *q, int64_t Hq, float scale, float *out, void *stream)
{
    int64_t cache_blocks;
    const int st = check_attn_shape(type, B, Hkv, Tc, D, T, Hq, &cache_blocks);
    if (st != TQ_OK)
        return st;
    if (B == 0)
        return TQ_OK;
    if (!k_codes || !k_norms || !v_codes || !v_norms || !q || !out)
        return TQ_ERR_NULL;
    if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q, 16) ||
        !aligned(k_norms, 2) || !aligned(v_norms, 2) || !aligned(out, 4))
        return TQ_ERR_ALIGN;
    if (tq::attn_workspace_bytes(type, B, Hkv, T, Hq, D / tq::kBlock) > TQ_ATTN_SCRATCH_BYTES)
        return TQ_ERR_WORKSPACE;
    const int64_t ob = B * Hq * D * 4, cb = cache_blocks * 16 * type, nb = cache_blocks * 2;
    const void *ins[5] = {k_codes, k_norms, v_codes, v_norms, q};
    const int64_t inb[5] = {cb, nb, cb, nb, B * Hq * D * 2};
    for (int i = 0; i < 5; ++i)
        if (overlap(out, ob, ins[i], inb[i]))
            return TQ_ERR_ALIAS;
    void *work = tq::attn_scratch();
    if (!work)
        return TQ_ERR_DEVICE;
    return tq::launch_attn(type, to_signs(signs), k_codes, k_norms, v_codes, v_norms, B, Hkv, Tc,
                           D / tq::kBlock, T, q, Hq, scale, out, work, stream)
               ? TQ_ERR_DEVICE
               : TQ_OK;
}
