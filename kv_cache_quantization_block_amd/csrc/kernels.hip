// kernels.hip -- gfx950 kernels of the turbo3 / turbo2 block codec.
//
// Method: "llama.cpp に TurboQuant を実装 -- 2bit・3bit の KV キャッシュ圧縮"
// (openalchemy.io).  Section "TurboQuant の何が違うのか": normalise by the
// block norm, rotate with the fast Walsh-Hadamard transform (adds and subtracts
// only, its own inverse up to a factor 128), quantise every coordinate with the
// N(0,1) Lloyd-Max codebook; decode looks the codes up and runs the same
// transform again.  Section "どこまで小さくなるのか": 128 values + one fp16 norm
// per block.  Section "現在の実装と、これから": decode to fp16 before attention,
// and the fused read that scores queries without materialising fp16 keys.
//
// Mapping on CDNA4 (wave64, 4 SIMDs x 16 lanes per CU, 160 KB LDS per CU):
//  * encode / decode: one wavefront owns 64 consecutive blocks, one per lane.
//    The 16 KB of fp16 values move between HBM and the wave with fully
//    coalesced 16-byte accesses (every load / store instruction covers 1 KB
//    contiguous) and are transposed through a wave-private, XOR-swizzled LDS
//    tile, so each lane then holds a whole block and all seven butterfly
//    stages run inside its registers with no cross-lane traffic.
//  * the first two butterfly stages of the encoder are done on the fp16
//    inputs with v_dot2_f32_f16 against (1, 1) / (1, -1): exact products,
//    float accumulation, the fp16 -> f32 conversion folded in.
//  * the quantiser is one clamp, three FMAs and a float -> int conversion per
//    value: an odd polynomial that crosses k exactly at the k-th positive
//    threshold maps t to 2^b/2 + g(t), whose floor is the code.
//  * decode reads stage-one (turbo3) or stage-two (turbo2) outputs straight
//    from a small LDS table indexed by 6 / 8 packed code bits.
//  * q.K: q . (H y) = (H q) . y since H is symmetric, so each query slice is
//    rotated once per workgroup and every key token is scored with a table
//    lookup and one FMA per (value, query head); the decoded key is never
//    formed.  Four lanes share one 128-value key block; a wave scores 16 key
//    rows of one kv head for up to four query heads at a time.
// Everything is float32 arithmetic; the packed-fp32 instructions are disabled
// at compile time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace tq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = kBlocksPerWave * kBlock * 2;   // 16 KB of fp16 per wave

// Wave-private LDS tile of 64 blocks x 256 B.  Chunk c (16 B) of block b sits
// at b*256 + ((c ^ (b & 15)) * 16): a row of 16 chunks (coalesced side) and a
// column of 8 consecutive blocks (per-lane side) both touch distinct banks.
__device__ __forceinline__ uint32_t swz(uint32_t blk, uint32_t chunk)
{
    return blk * 256u + ((chunk ^ (blk & 15u)) << 4);
}

// Reinterpret a 32-bit word as two fp16 values.  The word is taken by value:
// bit-casting an element of an ext_vector (w.y) directly reads element 0 with
// this compiler, so vector elements always go through a scalar first.
__device__ __forceinline__ h2_t as_h2(uint32_t word) { return __builtin_bit_cast(h2_t, word); }

// d = a.x * b.x + a.y * b.y + c in the three-operand VOP3P form (the compiler's
// accumulate-in-place form would need a register copy per result here).
// fp16 x (+-1) products are exact, the sum is a float.
__device__ __forceinline__ float dot2(h2_t a, h2_t b, float c)
{
    float d;
    asm("v_dot2_f32_f16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ float dot2(h2_t a, h2_t b)
{
    float d;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// Order LDS traffic between the lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// In-register butterflies of the stages with span h in [H0, H1).
template <int H0, int H1 = kBlock>
__device__ __forceinline__ void fwht_from(float (&u)[kBlock])
{
#pragma unroll
    for (int h = H0; h < H1; h <<= 1)
#pragma unroll
        for (int i = 0; i < kBlock; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                float a = u[j], b = u[j + h];
                u[j] = a + b;
                u[j + h] = a - b;
            }
}

// Cache block of x-block b: x row (lh, t) -> cache row (lh, t0 + t).
__device__ __forceinline__ int64_t cache_block(uint32_t b, uint32_t row_blocks,
                                               int64_t cache_row_blocks, int64_t t0_blocks)
{
    uint32_t lh = b / row_blocks;
    uint32_t r = b - lh * row_blocks;
    return (int64_t)lh * cache_row_blocks + t0_blocks + r;
}

// ---------------------------------------------------------------- encode

template <int BITS>
__global__ __launch_bounds__(256, 2) void encode_kernel(const uint8_t *__restrict__ x,
                                                     uint32_t nblocks, uint32_t row_blocks,
                                                     int64_t cache_row_blocks, int64_t t0_blocks,
                                                     uint8_t *__restrict__ codes,
                                                     uint16_t *__restrict__ norms, Codebook cb)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile_all[kWavesPerGroup][kTileBytes];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t b0 = (blockIdx.x * kWavesPerGroup + wave) * kBlocksPerWave;
    if (b0 >= nblocks)
        return;
    uint8_t *tile = tile_all[wave];
    const uint32_t nb = min(nblocks - b0, (uint32_t)kBlocksPerWave);

    // 1. coalesced 16-byte loads of the wave's 64 blocks, transposed through LDS
    {
        const uint8_t *src = x + (size_t)b0 * (kBlock * 2);
        u4_t r[16];
        if (nb == kBlocksPerWave) {   // full tile (wave-uniform): no per-load guard
#pragma unroll
            for (int k = 0; k < 16; ++k)
                r[k] = *(const u4_t *)(src + k * 1024 + lane * 16);
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                uint32_t blk = 4 * k + (lane >> 4);
                r[k] = blk < nb ? *(const u4_t *)(src + k * 1024 + lane * 16) : u4_t{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k)
            *(u4_t *)(tile + swz(4 * k + (lane >> 4), lane & 15u)) = r[k];
    }
    wave_lds_sync();
    h2_t v[64];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const u4_t w = *(const u4_t *)(tile + swz(lane, c));
        v[4 * c + 0] = as_h2(w.x);
        v[4 * c + 1] = as_h2(w.y);
        v[4 * c + 2] = as_h2(w.z);
        v[4 * c + 3] = as_h2(w.w);
    }

    // 2. norm: sum of squares with exact fp16 products, eight partial sums
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        acc[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k)
        acc[k & 7] = __builtin_amdgcn_fdot2(v[k], v[k], acc[k & 7], false);
    const float ss = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    const float n = __builtin_sqrtf(ss);

    // 3. rotation.  Stages of span 1 and 2 straight from the fp16 pairs, two
    //    results per input pair; the results at positions with bit 1 set come out
    //    negated (p - (x0 + x1) instead of (x0 + x1) - p), which saves the negation.
    //    Every later stage only combines positions that agree in bit 1, so after the
    //    remaining stages u[i] holds -(H x)[i] exactly wherever i & 2, and +(H x)[i]
    //    elsewhere (IEEE rounding is symmetric, the values are exact negations).
    float u[kBlock];
    {
        const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        const h2_t pm = {(_Float16)1.0f, (_Float16)-1.0f};
        const h2_t mm = {(_Float16)-1.0f, (_Float16)-1.0f};
        const h2_t mp = {(_Float16)-1.0f, (_Float16)1.0f};
#pragma unroll
        for (int g = 0; g < 32; ++g) {
            const float p = dot2(v[2 * g + 1], one);          //  x2 + x3
            const float q = dot2(v[2 * g + 1], pm);           //  x2 - x3
            u[4 * g + 0] = dot2(v[2 * g], one, p);            //  (x0 + x1) + (x2 + x3)
            u[4 * g + 1] = dot2(v[2 * g], pm, q);             //  (x0 - x1) + (x2 - x3)
            u[4 * g + 2] = dot2(v[2 * g], mm, p);             // -((x0 + x1) - (x2 + x3))
            u[4 * g + 3] = dot2(v[2 * g], mp, q);             // -((x0 - x1) - (x2 - x3))
        }
    }
    fwht_from<4>(u);

    // 4. quantise t = u / n:  F = 2^b/2 + g(clamp(t)), code = floor(F).  The
    //    polynomial's coefficients absorb 1/n and the clamp is scaled by n, so the
    //    division is never done per value; g is odd, so a negated u[i] is handled
    //    by negating the last product (bit-identical to quantising +(H x)[i]).
    //    n == 0 (zero block) gives F = 2^b/2 for every value.
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    const float k1 = cb.g1 * rn, k2 = cb.g2 * rn * rn, k3 = cb.g3 * rn * rn * rn;
    const float hi = cb.clamp_t * n, lo = -hi;
    constexpr float mid = (float)(1 << (BITS - 1));
    constexpr int NW = 4 * BITS;   // 32-bit words of packed codes per block
    uint32_t w[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k)
        w[k] = 0u;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
        const float uc = __builtin_amdgcn_fmed3f(u[i], lo, hi);
        const float ui = (i & 2) ? -uc : uc;
        float F;
        if constexpr (BITS == 3) {
            // g(t) = t * (g1 + g2 |t| + g3 t^2)
            float p = __builtin_fmaf(__builtin_fabsf(uc), k3, k2);
            p = __builtin_fmaf(__builtin_fabsf(uc), p, k1);
            F = __builtin_fmaf(ui, p, mid);
        } else {
            F = __builtin_fmaf(ui, k1, mid);
        }
        const uint32_t code = (uint32_t)F;
        const int bit = BITS * i, wi = bit >> 5, sh = bit & 31;
        w[wi] |= code << sh;
        if (sh + BITS > 32)
            w[wi + 1] |= code >> (32 - sh);
    }

    // 5. store codes (16*BITS bytes) and the fp16 norm of this lane's block
    const uint32_t b = b0 + lane;
    if (b < nblocks) {
        const int64_t dst = cache_block(b, row_blocks, cache_row_blocks, t0_blocks);
        u4_t *out = (u4_t *)(codes + dst * (16 * BITS));
#pragma unroll
        for (int k = 0; k < BITS; ++k)
            out[k] = u4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
        const _Float16 n16 = (_Float16)__builtin_fminf(n, 65504.0f);
        norms[dst] = __builtin_bit_cast(uint16_t, n16);
    }
}

// ---------------------------------------------------------------- decode

template <int BITS>
__global__ __launch_bounds__(256) void decode_kernel(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ norms,
                                                     uint32_t nblocks, uint32_t row_blocks,
                                                     int64_t cache_row_blocks, int64_t t0_blocks,
                                                     uint8_t *__restrict__ x, Codebook cb)
{
    // turbo3: 64 entries (6 code bits = two codes) -> stage-one outputs (y0+y1, y0-y1)
    // turbo2: 256 entries (8 code bits = four codes) -> stage-two outputs
    constexpr int NE = BITS == 3 ? 64 : 256;
    constexpr int EW = BITS == 3 ? 2 : 4;
    constexpr int kTableBytes = NE * EW * 4;
    // one LDS buffer, the table first: its entries are then addressed by the
    // extracted code bits alone (the 16-bit instruction offset cannot reach past
    // the 64 KB of tiles)
    __shared__ __attribute__((aligned(16))) uint8_t smem[kTableBytes + kWavesPerGroup * kTileBytes];
    float *table = (float *)smem;
    for (int e = threadIdx.x; e < NE; e += blockDim.x) {
        if constexpr (BITS == 3) {
            float y0 = cb.levels[e & 7], y1 = cb.levels[e >> 3];
            table[2 * e] = y0 + y1;
            table[2 * e + 1] = y0 - y1;
        } else {
            float y0 = cb.levels[e & 3], y1 = cb.levels[(e >> 2) & 3];
            float y2 = cb.levels[(e >> 4) & 3], y3 = cb.levels[e >> 6];
            float s0 = y0 + y1, s1 = y0 - y1, s2 = y2 + y3, s3 = y2 - y3;
            table[4 * e] = s0 + s2;
            table[4 * e + 1] = s1 + s3;
            table[4 * e + 2] = s0 - s2;
            table[4 * e + 3] = s1 - s3;
        }
    }
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t b0 = (blockIdx.x * kWavesPerGroup + wave) * kBlocksPerWave;
    if (b0 >= nblocks)
        return;
    uint8_t *tile = smem + kTableBytes + wave * kTileBytes;
    const uint32_t nb = min(nblocks - b0, (uint32_t)kBlocksPerWave);
    const uint32_t b = b0 + lane;
    const bool valid = b < nblocks;

    constexpr int NW = 4 * BITS;
    uint32_t w[NW];
    float scale = 0.0f;
    if (valid) {
        const int64_t src = cache_block(b, row_blocks, cache_row_blocks, t0_blocks);
        const u4_t *in = (const u4_t *)(codes + src * (16 * BITS));
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
            u4_t c = in[k];
            w[4 * k] = c.x;
            w[4 * k + 1] = c.y;
            w[4 * k + 2] = c.z;
            w[4 * k + 3] = c.w;
        }
        scale = (float)__builtin_bit_cast(_Float16, norms[src]) * (1.0f / 128.0f);
    } else {
#pragma unroll
        for (int k = 0; k < NW; ++k)
            w[k] = 0u;
    }

    float u[kBlock];
    if constexpr (BITS == 3) {
#pragma unroll
        for (int p = 0; p < 64; ++p) {
            const int bit = 6 * p, wi = bit >> 5, sh = bit & 31;
            uint32_t e = sh <= 26 ? (w[wi] >> sh) & 63u
                                  : __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 63u;
            float2 t = *(const float2 *)(table + 2 * e);
            u[2 * p] = t.x;
            u[2 * p + 1] = t.y;
        }
        fwht_from<2, 64>(u);
    } else {
#pragma unroll
        for (int p = 0; p < 32; ++p) {
            uint32_t e = (w[p >> 2] >> (8 * (p & 3))) & 255u;
            float4 t = *(const float4 *)(table + 4 * e);
            u[4 * p] = t.x;
            u[4 * p + 1] = t.y;
            u[4 * p + 2] = t.z;
            u[4 * p + 3] = t.w;
        }
        fwht_from<4, 64>(u);
    }
    // last stage with the rescale by n16/128 folded in: (a +- b) s = a s +- b s
#pragma unroll
    for (int j = 0; j < 64; ++j) {
        const float as = u[j] * scale, bj = u[j + 64];
        u[j] = __builtin_fmaf(bj, scale, as);
        u[j + 64] = __builtin_fmaf(-bj, scale, as);
    }

    // round to fp16 (nearest even) and transpose back through LDS
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            h2_t hv = {(_Float16)u[8 * c + 2 * k], (_Float16)u[8 * c + 2 * k + 1]};
            o[k] = __builtin_bit_cast(uint32_t, hv);
        }
        *(u4_t *)(tile + swz(lane, c)) = u4_t{o[0], o[1], o[2], o[3]};
    }
    wave_lds_sync();
    uint8_t *dst = x + (size_t)b0 * (kBlock * 2);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        uint32_t blk = 4 * k + (lane >> 4);
        u4_t r = *(const u4_t *)(tile + swz(blk, lane & 15u));
        if (blk < nb)
            *(u4_t *)(dst + k * 1024 + lane * 16) = r;
    }
}

// ---------------------------------------------------------------- q.K scores

constexpr int kQkTokensPerGroup = 1024;

// BITS: 2 or 3.  GH: query heads per pass (1, 2 or 4).  LPT: lanes per key token
// (4 * next power of two of m); lane = token * LPT + slice * 4 + part, the lane
// covers values [32*part, 32*part + 32) of 128-block `slice` of the token.
template <int BITS, int GH>
__global__ __launch_bounds__(256) void qk_kernel(const uint8_t *__restrict__ k_codes,
                                                 const uint16_t *__restrict__ k_norms,
                                                 const uint16_t *__restrict__ q,
                                                 float *__restrict__ scores, uint32_t Hkv,
                                                 int64_t Tc, uint32_t T, uint32_t m,
                                                 uint32_t lpt_log2, uint32_t G, uint32_t Hq,
                                                 uint32_t passes, float scale, Codebook cb)
{
    // turbo3: 64 entries (two codes) -> (y0, y1); turbo2: 256 entries (four codes) -> y0..y3
    constexpr int NE = BITS == 3 ? 64 : 256;
    constexpr int EW = BITS == 3 ? 2 : 4;
    constexpr int kTableFloats = NE * EW;
    // one LDS buffer, the lookup table first (addressed by code bits alone), then
    // the rotated query slices qs[head * m + slice][i]
    __shared__ __attribute__((aligned(16))) float smem[kTableFloats + GH * 16 * kBlock];
    float *table = smem;
    float(*qs)[kBlock] = (float(*)[kBlock])(smem + kTableFloats);

    const uint32_t pass = blockIdx.x % passes;
    const uint32_t bg = blockIdx.x / passes;           // b * Hkv + g
    const uint32_t b = bg / Hkv, g = bg - b * Hkv;
    const uint32_t h0 = g * G + pass * GH;             // first query head of this pass

    for (int e = threadIdx.x; e < NE; e += blockDim.x) {
        if constexpr (BITS == 3) {
            table[2 * e] = cb.levels[e & 7];
            table[2 * e + 1] = cb.levels[e >> 3];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                table[4 * e + k] = cb.levels[(e >> (2 * k)) & 3];
        }
    }
    // load the GH x m query slices as float, then rotate each in place
    const uint32_t nvec = GH * m;
    for (uint32_t i = threadIdx.x; i < nvec * kBlock; i += blockDim.x) {
        uint32_t r = i / (m * kBlock), rest = i - r * (m * kBlock);
        uint16_t hq = q[((size_t)b * Hq + h0 + r) * (m * kBlock) + rest];
        qs[r * m + rest / kBlock][rest % kBlock] = (float)__builtin_bit_cast(_Float16, hq);
    }
    __syncthreads();
    for (uint32_t h = 1; h < kBlock; h <<= 1) {
        for (uint32_t p = threadIdx.x; p < nvec * (kBlock / 2); p += blockDim.x) {
            uint32_t vec = p / (kBlock / 2), i = p % (kBlock / 2);
            uint32_t j = (i / h) * 2 * h + (i % h);
            float a = qs[vec][j], c = qs[vec][j + h];
            qs[vec][j] = a + c;
            qs[vec][j + h] = a - c;
        }
        __syncthreads();
    }

    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t lpt = 1u << lpt_log2, tpw = 64u >> lpt_log2;
    const uint32_t tok = lane >> lpt_log2, sub = lane & (lpt - 1u);
    const uint32_t slice = sub >> 2, part = sub & 3u;
    const bool active = slice < m;
    float qr[GH][32];
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int i = 0; i < 32; ++i)
            qr[h][i] = active ? qs[h * m + slice][32 * part + i] : 0.0f;

    const uint32_t t_begin = blockIdx.y * kQkTokensPerGroup;
    const uint32_t t_end = min(T, t_begin + kQkTokensPerGroup);
    const size_t row0 = (size_t)bg * Tc;                // first cache row of (b, g)
    constexpr int CB = 16 * BITS;                        // code bytes per block
    constexpr int LW = BITS;                             // 32-bit words per lane (32 codes)

    for (uint32_t tb = t_begin + wave * tpw; tb < t_end; tb += kWavesPerGroup * tpw) {
        const uint32_t t = tb + tok;
        const bool live = active && t < t_end;
        uint32_t w[LW];
        float f = 0.0f;
        if (live) {
            const size_t blk = (row0 + t) * m + slice;
            const uint32_t *src = (const uint32_t *)(k_codes + blk * CB + part * (4 * BITS));
#pragma unroll
            for (int k = 0; k < LW; ++k)
                w[k] = src[k];
            f = (float)__builtin_bit_cast(_Float16, k_norms[blk]) * (1.0f / 128.0f);
        } else {
#pragma unroll
            for (int k = 0; k < LW; ++k)
                w[k] = 0u;
        }
        float acc[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h)
            acc[h] = 0.0f;
        if constexpr (BITS == 3) {
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const int bit = 6 * p, wi = bit >> 5, sh = bit & 31;
                uint32_t e = sh <= 26 ? (w[wi] >> sh) & 63u
                                      : __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 63u;
                float2 y = *(const float2 *)(table + 2 * e);
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    acc[h] = __builtin_fmaf(qr[h][2 * p], y.x, acc[h]);
                    acc[h] = __builtin_fmaf(qr[h][2 * p + 1], y.y, acc[h]);
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                uint32_t e = (w[p >> 2] >> (8 * (p & 3))) & 255u;
                float4 y = *(const float4 *)(table + 4 * e);
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    acc[h] = __builtin_fmaf(qr[h][4 * p], y.x, acc[h]);
                    acc[h] = __builtin_fmaf(qr[h][4 * p + 1], y.y, acc[h]);
                    acc[h] = __builtin_fmaf(qr[h][4 * p + 2], y.z, acc[h]);
                    acc[h] = __builtin_fmaf(qr[h][4 * p + 3], y.w, acc[h]);
                }
            }
        }
        // per-slice norm, then sum the LPT lanes of the token
#pragma unroll
        for (int h = 0; h < GH; ++h)
            acc[h] *= f;
        for (uint32_t s = 1; s < lpt; s <<= 1)
#pragma unroll
            for (int h = 0; h < GH; ++h)
                acc[h] += __shfl_xor(acc[h], (int)s, 64);
        if (t < t_end && sub < GH) {
            float r = acc[0];
#pragma unroll
            for (int h = 1; h < GH; ++h)
                r = sub == (uint32_t)h ? acc[h] : r;
            scores[((size_t)b * Hq + h0 + sub) * T + t] = scale * r;
        }
    }
}

inline int grid_for(int64_t nblocks)
{
    int64_t per_group = (int64_t)kWavesPerGroup * kBlocksPerWave;
    return (int)((nblocks + per_group - 1) / per_group);
}

}  // namespace

int launch_encode(int bits, const void *x, int64_t nblocks, int64_t row_blocks,
                  int64_t cache_row_blocks, int64_t t0_blocks, void *codes, void *norms,
                  void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    dim3 grid(grid_for(nblocks)), block(256);
    if (bits == 3)
        hipLaunchKernelGGL(encode_kernel<3>, grid, block, 0, s, (const uint8_t *)x,
                           (uint32_t)nblocks, (uint32_t)row_blocks, cache_row_blocks, t0_blocks,
                           (uint8_t *)codes, (uint16_t *)norms, *cb);
    else
        hipLaunchKernelGGL(encode_kernel<2>, grid, block, 0, s, (const uint8_t *)x,
                           (uint32_t)nblocks, (uint32_t)row_blocks, cache_row_blocks, t0_blocks,
                           (uint8_t *)codes, (uint16_t *)norms, *cb);
    return (int)hipGetLastError();
}

int launch_decode(int bits, const void *codes, const void *norms, int64_t nblocks,
                  int64_t row_blocks, int64_t cache_row_blocks, int64_t t0_blocks, void *x,
                  void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    dim3 grid(grid_for(nblocks)), block(256);
    if (bits == 3)
        hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, s, (const uint8_t *)codes,
                           (const uint16_t *)norms, (uint32_t)nblocks, (uint32_t)row_blocks,
                           cache_row_blocks, t0_blocks, (uint8_t *)x, *cb);
    else
        hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, s, (const uint8_t *)codes,
                           (const uint16_t *)norms, (uint32_t)nblocks, (uint32_t)row_blocks,
                           cache_row_blocks, t0_blocks, (uint8_t *)x, *cb);
    return (int)hipGetLastError();
}

int launch_qk(int bits, const void *k_codes, const void *k_norms, int64_t B, int64_t Hkv,
              int64_t Tc, int64_t m, int64_t T, const void *q, int64_t Hq, float scale,
              float *scores, void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    const int64_t G = Hq / Hkv;
    const int GH = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
    const int64_t passes = G / GH;
    uint32_t mp = 1, lpt_log2 = 2;
    while (mp < (uint32_t)m) {
        mp <<= 1;
        ++lpt_log2;
    }
    dim3 grid((uint32_t)(B * Hkv * passes), (uint32_t)((T + kQkTokensPerGroup - 1) / kQkTokensPerGroup));
    dim3 block(256);
#define TQ_QK_LAUNCH(BB, GG)                                                                    \
    hipLaunchKernelGGL((qk_kernel<BB, GG>), grid, block, 0, s, (const uint8_t *)k_codes,        \
                       (const uint16_t *)k_norms, (const uint16_t *)q, scores, (uint32_t)Hkv,   \
                       Tc, (uint32_t)T, (uint32_t)m, lpt_log2, (uint32_t)G, (uint32_t)Hq,      \
                       (uint32_t)passes, scale, *cb)
    if (bits == 3) {
        if (GH == 4) TQ_QK_LAUNCH(3, 4);
        else if (GH == 2) TQ_QK_LAUNCH(3, 2);
        else TQ_QK_LAUNCH(3, 1);
    } else {
        if (GH == 4) TQ_QK_LAUNCH(2, 4);
        else if (GH == 2) TQ_QK_LAUNCH(2, 2);
        else TQ_QK_LAUNCH(2, 1);
    }
#undef TQ_QK_LAUNCH
    return (int)hipGetLastError();
}

}  // namespace tq
