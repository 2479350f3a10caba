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
// Mapping on CDNA4 (wave64, 4 SIMDs x 16 lanes per CU, 160 KB LDS per CU, matrix
// cores per SIMD):
//  * encode: a wave owns 32 consecutive blocks.  The rotation's H_32 factor runs on
//    the matrix cores straight from the fp16 loads (+-1 weights: exact products,
//    fp32 sums), the H_4 factor as two butterfly stages in registers; the norm's
//    sum of squares comes from the same registers by v_dot2.
//  * the quantiser is one clamp and three FMAs per value (turbo2: one): an odd
//    polynomial that crosses k exactly at the k-th positive threshold maps t to
//    2^b/2 + g(t), whose floor is the code; the last FMA adds 2^23 under
//    round-toward-minus-infinity, which leaves the floor in the low mantissa
//    bits, and eight codes are then packed by seven shift-adds.
//  * decode: the same factorisation run backwards.  A wave owns 32 blocks; the
//    levels, looked up two codes at a time in a small LDS table as fp16 hi / lo
//    pairs, enter the H_32 products as the B operand, H_4 and the rescale run in
//    registers, and the fp16 output leaves through an XOR-swizzled LDS stage as
//    16-byte stores, 1 KB contiguous per instruction.
//  * q.K: q . (H y) = (H q) . y since H is symmetric, so each query slice is rotated
//    once per workgroup and the keys' levels enter v_mfma_f32_16x16x32_f16 as fp16
//    hi / lo pairs read from an LDS table; the decoded key is never formed.
//  * decode attention: the same scores, an online softmax per batch of 64 / m rows
//    (m blocks per row) and P.V on the matrix cores in the rotated domain, one
//    inverse transform per head at the end of a second (combine) pass over per-chunk
//    partials.
//  * both fused read kernels give every wave an equal share of rows and raise the
//    priority of the waves with the most work left, so that the arbiters' preference
//    for older waves does not leave a tail of late ones.
//  * interleaved records: LDS-staged 16-byte moves between the planes and the
//    50 / 34-byte block records.
//  * the randomised rotation H D flips fp16 sign bits (XOR) where the kernels load
//    or store values, and the query and the attention output where they enter and
//    leave.
// Arithmetic is float32, except the matrix-core operands (fp16 inputs, fp16 hi / lo
// splits of float values); the packed-fp32 instructions are disabled at compile
// time.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <atomic>
#include <stdint.h>
#include <stdlib.h>

#include "internal.h"
#include "tq.h"

namespace tq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));   // a matrix-core fp16 operand
typedef float f4_t __attribute__((ext_vector_type(4)));      // a 16 x 16 product's four rows

// Wave-private LDS tile of fp16 blocks, 256 B each.  Chunk c (16 B) of block b sits
// at b*256 + ((c ^ (b & 15)) * 16): 16 lanes writing one chunk of 16 consecutive
// blocks, and 16 lanes reading the 16 chunks of one block, both touch distinct banks.
__device__ __forceinline__ uint32_t swz(uint32_t blk, uint32_t chunk)
{
    return blk * 256u + ((chunk ^ (blk & 15u)) << 4);
}

// Reinterpret a 32-bit word as two fp16 values.  The word is taken by value:
// bit-casting an element of an ext_vector (w.y) directly reads element 0 with
// this compiler, so vector elements always go through a scalar first.
__device__ __forceinline__ h2_t as_h2(uint32_t word) { return __builtin_bit_cast(h2_t, word); }

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b)
{
    return __builtin_bit_cast(uint32_t, h2_t{a, b});
}

// x = hi + lo with hi = fp16(x), lo = fp16(x - hi) (x - hi is exact in float).
__device__ __forceinline__ void split_f16(float x, _Float16 &hi, _Float16 &lo)
{
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

// Streaming global accesses.  Each call reads its inputs (fp16 K/V, codes, norms)
// exactly once, so those loads carry the non-temporal hint: they do not allocate
// in the 256 MB memory-side cache, where an allocation that evicts a dirty line
// costs a write-back inside this kernel.  The encoder's codes and norms are read
// back much later (by decode or q.K of later steps), so they are stored with the
// hint too and leave no dirty lines behind.  Decoded fp16 values and scores are
// consumed by the very next kernel (attention, softmax) and use plain stores,
// which also stream large outputs at a higher rate than hinted stores do.
template <class T>
__device__ __forceinline__ T ld_stream(const T *p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_stream(T *p, T v) { __builtin_nontemporal_store(v, p); }

// LDS by integer address (the byte offset in the workgroup's LDS).
typedef __attribute__((address_space(3))) uint8_t lds_u8;
template <class T>
__device__ __forceinline__ T lds_load(uint32_t addr)
{
    return *(__attribute__((address_space(3))) const T *)(uintptr_t)addr;
}

// Lookup tables of 8-byte entries are replicated kLdsCopies8 times: the LDS serves
// 256 bytes (32 lanes x 8 B) per cycle from 64 banks, so the 32 lanes of one cycle,
// each reading its own copy, never collide whatever entries they pick.
constexpr int kLdsCopies8 = 32;

// Threads of every workgroup these kernels launch with.  Loops step by this constant,
// not by blockDim.x: reading blockDim.x is a load from the dispatch packet, and the
// wait for it would also wait for every load issued before it (loads complete in order).
constexpr uint32_t kGroupThreads = kWavesPerGroup * kWave;


// The value of another lane of the same quad (DPP quad_perm pattern CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Max / sum over each row of 16 lanes, one DPP ALU instruction per step (the builtin
// route adds a zeroing move and a canonicalising max to each step).  Two wait states
// precede each DPP read of a VGPR that a VALU instruction may just have written.
__device__ __forceinline__ float row16_max(float x)
{
    float r;
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "=&v"(r)
        : "v"(x));
    return r;
}
__device__ __forceinline__ float row16_sum(float x)
{
    float r;
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "=&v"(r)
        : "v"(x));
    return r;
}

// (a << S) + b as one v_lshl_add_u32 (kept as written: the compiler would otherwise
// re-associate a chain of these into more instructions).
template <int S>
__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "i"(S), "v"(b));
    return d;
}

// Float rounding mode of this wave (MODE.FP_ROUND, single-precision field).
__device__ __forceinline__ void set_f32_round_down() { __builtin_amdgcn_s_setreg(0x801, 2); }
__device__ __forceinline__ void set_f32_round_nearest() { __builtin_amdgcn_s_setreg(0x801, 0); }

// Pins values in registers at this point of the program: an empty volatile asm that
// takes and returns them.  Volatile asm keeps its order relative to the mode-register
// writes, so values pinned after set_f32_round_down() are computed after it and values
// pinned before set_f32_round_nearest() are computed before it.
__device__ __forceinline__ void pin4(float (&v)[4])
{
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

// F[i] = floor(x[i] * y[i] + M) + 2^23 as a float (its low mantissa bits hold the
// integer), for 0 <= x * y + M < 2^23: the FMA adds 2^23 + M, whose sum is a float of
// spacing 1, under round-toward-minus-infinity.  Only these four FMAs run in that mode;
// their operands are computed before it is set (in round-to-nearest) and their results
// are pinned before it is cleared.
template <int M>
__device__ __forceinline__ void round_down_fma4(float (&x)[4], float (&y)[4], float (&F)[4])
{
    constexpr float magic = 8388608.0f + (float)M;   // 2^23 + M, exact
    pin4(x);
    pin4(y);
    set_f32_round_down();
    float a[4] = {x[0], x[1], x[2], x[3]}, b[4] = {y[0], y[1], y[2], y[3]};
    pin4(a);
    pin4(b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        F[i] = __builtin_fmaf(a[i], b[i], magic);
    pin4(F);
    set_f32_round_nearest();
}

// The codebook levels into LDS.  Indexing the kernel-argument copy with a per-lane
// index would turn every table entry into a round trip to memory; one lane copies
// the levels with constant indices (scalar loads) and the caller barriers.
__device__ __forceinline__ void levels_to_lds(float *lv, const Codebook &cb)
{
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            lv[k] = cb.levels[k];
    }
}

// Wave priority by the work a wave has left.  The fused read kernels split their rows
// statically, one equal share per wave, and the SIMDs' arbiters favour older waves: with
// every wave at the same priority, waves of equal work finish up to 1.6x apart (at the
// 16-sequence decode step, q.K's waves took 37-60 us and the attention's 80-123 us), and
// a launch lasts as long as its slowest wave.  Giving the waves with more work left the
// higher priority lets the lagging waves issue first and keeps all of them in step
// (spans 60 -> 56 us and 120 -> 112 us; all waves end within the last eighth of the work).
// Called once per batch with the batch index and the batch count; wave-uniform.
__device__ __forceinline__ void prio_by_progress(uint32_t done, uint32_t total)
{
    const uint32_t rem = total - done;
    if (rem * 2u > total)
        __builtin_amdgcn_s_setprio(3);
    else if (rem * 4u > total)
        __builtin_amdgcn_s_setprio(2);
    else if (rem * 8u > total)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Order LDS traffic between the lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cache block of x-block b: x row (lh, t) -> cache row (lh, t0 + t).
__device__ __forceinline__ int64_t cache_block(uint32_t b, uint32_t row_blocks,
                                               int64_t cache_row_blocks, int64_t t0_blocks)
{
    uint32_t lh = b / row_blocks;
    uint32_t r = b - lh * row_blocks;
    return (int64_t)lh * cache_row_blocks + t0_blocks + r;
}

// Codec wave tiles: 32 consecutive blocks (the last one may be short), two 16-block
// column tiles of the matrix-core rotation (encode and decode).  Wave w handles tiles
// w, w + W, w + 2W... (W = waves in the grid); the grid normally gives every wave
// one tile (an encode wave with several prefetches tile i + W while it computes i).
constexpr int kEncTileBlocks = 32;

// (upper 32 lanes of a) <-> (lower 32 lanes of b), returned as the new (a, b).
__device__ __forceinline__ void swap32(float &a, float &b)
{
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                              __builtin_bit_cast(uint32_t, b), false, false);
    const uint32_t r0 = r[0], r1 = r[1];   // through scalars: see as_h2
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}

// Signs of the randomised rotation H D.  Word k of the kernel argument is read with
// a constant index (a per-lane index would load the argument through memory).
__device__ __forceinline__ uint32_t sign_word(const Signs &sg, uint32_t k)
{
    const uint32_t lo = k & 1u ? sg.w[1] : sg.w[0], hi = k & 1u ? sg.w[3] : sg.w[2];
    return k & 2u ? hi : lo;
}
// fp16 sign-flip masks of the eight positions 8 c .. 8 c + 7 (one 16-byte chunk of a
// block, as four packed pairs): XOR with them applies D to the chunk.
__device__ __forceinline__ u4_t sign_mask_chunk(const Signs &sg, uint32_t c)
{
    const uint32_t byte = sign_word(sg, c >> 2) >> (8u * (c & 3u));
    u4_t m;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m[j] = (((byte >> (2 * j)) & 1u) << 15) | (((byte >> (2 * j + 1)) & 1u) << 31);
    return m;
}
// float sign-flip mask of position p < 128.
__device__ __forceinline__ uint32_t sign_mask_f32(const Signs &sg, uint32_t p)
{
    return ((sign_word(sg, p >> 5) >> (p & 31u)) & 1u) << 31;
}

// Writes a finished tile: packed codes staged in LDS (block b at b * 16 * BITS)
// and each lane's norm.  Consecutive cache blocks (always, unless the tile
// straddles two (layer, head) rows of a cache longer than x) leave as contiguous
// 16-byte stores; otherwise every lane writes its two 32-code groups itself.
template <int BITS>
__device__ __forceinline__ void store_enc_tile(const uint8_t *stage, uint32_t lane, uint32_t b0,
                                               uint32_t nb, uint16_t n16, uint32_t row_blocks,
                                               int64_t cache_row_blocks, int64_t t0_blocks,
                                               uint8_t *__restrict__ codes,
                                               uint16_t *__restrict__ norms)
{
    constexpr int GW = BITS, GB = 4 * BITS, CB = 16 * BITS;
    const uint32_t blk = lane & 31u, half = lane >> 5;
    // consecutive cache blocks: always when the cache rows hold exactly the encoded
    // rows (no division needed), else when the tile stays inside one cache row
    const bool contig = cache_row_blocks == (int64_t)row_blocks && t0_blocks == 0;
    const int64_t dst0 = contig ? (int64_t)b0 : cache_block(b0, row_blocks, cache_row_blocks, t0_blocks);
    if (contig ||
        cache_block(b0 + nb - 1, row_blocks, cache_row_blocks, t0_blocks) - dst0 == (int64_t)nb - 1) {
        uint8_t *gdst = codes + dst0 * CB;
        const uint32_t nchunks = nb * BITS;   // 16-byte chunks of the tile's codes
#pragma unroll
        for (int k = 0; k < (2 * BITS + 3) / 4; ++k) {
            const uint32_t c = k * 64 + lane;
            if (c < 2u * BITS * 16u) {
                const u4_t val = *(const u4_t *)(stage + c * 16);
                if (c < nchunks)
                    st_stream((u4_t *)(gdst + c * 16), val);
            }
        }
        if (blk < nb && half == 0)
            st_stream(norms + dst0 + blk, n16);
    } else if (blk < nb) {
        const int64_t dst = cache_block(b0 + blk, row_blocks, cache_row_blocks, t0_blocks);
        const uint32_t *src = (const uint32_t *)(stage + blk * CB + GB * half);
        uint32_t *out = (uint32_t *)(codes + dst * CB + GB * half);
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            st_stream(out + k, src[k]);
            st_stream(out + 2 * GW + k, src[2 * GW + k]);
        }
        if (half == 0)
            st_stream(norms + dst, n16);
    }
}

// ---------------------------------------------------------------- encode
//
// The rotation u = H x is a dense contraction with a +-1 matrix, and Sylvester's H
// factors over the index split p = 32 g + q as H_128 = H_4 (x) H_32:
//   v_g'[q]     = sum_q' H_32[q][q'] x[32 g' + q']     (matrix cores, v_mfma_f32_16x16x32_f16:
//                                                        fp16 inputs, +-1 weights, exact
//                                                        products summed in fp32)
//   u[32 g + q] = sum_g' H_4[g][g'] v_g'[q]             (two butterfly stages per value)
// which replaces the seven butterfly stages of the VALU encoder by two.  A wave takes
// 32 blocks as two 16-block column tiles.  Column n of a product is block 16 c + n;
// the k-slots of lane group G (lane / 16) are values 32 g' + 8 G .. + 7 of that block,
// one 16-byte load that is the B operand as loaded.  Row i of row tile r is H_32 row
// 8 (i / 4) + 4 r + i % 4, so lane group G receives q = 8 G .. 8 G + 7 of every g':
// after the butterflies it holds positions 32 g + 8 G .. + 7 for g = 0..3, four runs of
// eight codes (24 / 16 bits, byte aligned), which go to the staged tile by byte writes.
// The norm's sum of squares comes from the same loads (v_dot2 of exact fp16 squares)
// and is summed over the four lane groups of a block in one fixed order.
// LOOP: the grid may give a wave several tiles (false: one tile per wave, so nothing
// is prefetched for a next one).
template <int BITS, bool ROT, bool LOOP>
__global__ __launch_bounds__(256, 3) void encode_kernel(const uint8_t *__restrict__ x,
                                                            uint32_t nblocks, uint32_t row_blocks,
                                                            int64_t cache_row_blocks,
                                                            int64_t t0_blocks,
                                                            uint8_t *__restrict__ codes,
                                                            uint16_t *__restrict__ norms,
                                                            Codebook cb, Signs sg)
{
    constexpr int CB = 16 * BITS;         // code bytes per block
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWavesPerGroup][kEncTileBlocks * 48];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n = lane & 15u, G = lane >> 4;
    const uint32_t ntiles = (nblocks + kEncTileBlocks - 1) / kEncTileBlocks;
    const uint32_t stride = gridDim.x * kWavesPerGroup;
    uint32_t tile = blockIdx.x * kWavesPerGroup + wave;
    // turbo2 with one tile per wave: in each whole run of 32 tiles (8 workgroups, which
    // the dispatcher deals to the 8 XCDs in turn) tile 8 w + x goes to wave w of the
    // run's x-th workgroup, so consecutive 8 KB tiles sit on different XCDs.  turbo2
    // measured 1.5-3 % faster so, turbo3 0.4-1.3 % slower, and keeps the plain order.
    if constexpr (BITS == 2) {
        if (gridDim.x * kWavesPerGroup >= ntiles && (tile | 31u) < ntiles)
            tile = (tile & ~31u) + wave * 8u + (blockIdx.x & 7u);
    }
    if (tile >= ntiles)
        return;
    uint8_t *stage = stage_all[wave];

    // loads of column tile c of a tile: R[c][g'] = values 32 g' + 8 G .. + 7 of block
    // b0 + 16 c + n; lanes past the tile's blocks read its last block (their codes and
    // norms are never stored), so every load is unconditional
    u4_t R[2][4];
    auto load_col = [&](uint32_t t, int c) {
        const uint32_t b0 = t * kEncTileBlocks;
        const uint32_t nb = min(nblocks - b0, (uint32_t)kEncTileBlocks);
        const uint32_t b = min(16u * c + n, nb - 1u);
        const u4_t *src = (const u4_t *)(x + ((size_t)b0 + b) * (kBlock * 2) + 16u * G);
#pragma unroll
        for (int gp = 0; gp < 4; ++gp)
            R[c][gp] = ld_stream(src + 4 * gp);
    };
    load_col(tile, 0);   // the first tile's loads go out before the operand set-up
    load_col(tile, 1);
    // A operands: row tile r, lane row n -> H_32 row q = 8 (n / 4) + 4 r + n % 4, k-slots
    // 8 G + s: +-1 as fp16 (sign bit of (-1)^popcount(q & k))
    h8_t A[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint32_t q = 8u * (n >> 2) + 4u * r + (n & 3u);
        uint32_t w[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const uint32_t k0 = 8u * G + 2u * s2;
            const uint32_t h0 = (__builtin_popcount(q & k0) & 1u) ? 0xBC00u : 0x3C00u;
            const uint32_t h1 = (__builtin_popcount(q & (k0 + 1u)) & 1u) ? 0xBC00u : 0x3C00u;
            w[s2] = h0 | (h1 << 16);
        }
        A[r] = __builtin_bit_cast(h8_t, u4_t{w[0], w[1], w[2], w[3]});
    }
    // randomised rotation: the chunk of load (c, g') is 4 g' + G of its block
    u4_t smask[4];
#pragma unroll
    for (int gp = 0; gp < 4; ++gp)
        smask[gp] = ROT ? sign_mask_chunk(sg, 4u * gp + G) : u4_t{0, 0, 0, 0};

    uint32_t pb0 = 0, pnb = 0;   // the finished tile waiting in `stage`
    uint16_t pn16 = 0;
    for (;;) {
        const uint32_t b0 = tile * kEncTileBlocks;
        const uint32_t nb = min(nblocks - b0, (uint32_t)kEncTileBlocks);
        const uint32_t next = LOOP ? tile + stride : ntiles;
        float nrm[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // 1. products v_g' of this column tile and its sums of squares, then the
            //    next tile's loads into the same registers
            f4_t D[4][2];
            float acc[2] = {0.0f, 0.0f};
#pragma unroll
            for (int gp = 0; gp < 4; ++gp) {
                const u4_t xv = ROT ? R[c][gp] ^ smask[gp] : R[c][gp];
                const h8_t B = __builtin_bit_cast(h8_t, xv);
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    D[gp][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A[r], B, f4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                acc[0] = __builtin_amdgcn_fdot2(as_h2(xv.x), as_h2(xv.x), acc[0], false);
                acc[1] = __builtin_amdgcn_fdot2(as_h2(xv.y), as_h2(xv.y), acc[1], false);
                acc[0] = __builtin_amdgcn_fdot2(as_h2(xv.z), as_h2(xv.z), acc[0], false);
                acc[1] = __builtin_amdgcn_fdot2(as_h2(xv.w), as_h2(xv.w), acc[1], false);
            }
            if (next < ntiles)
                load_col(next, c);
            if (c == 0) {   // 2. write out the previous tile before its bytes are reused
                if (pnb)
                    store_enc_tile<BITS>(stage, lane, pb0, pnb, pn16, row_blocks, cache_row_blocks,
                                         t0_blocks, codes, norms);
                wave_lds_sync();
            }

            // 3. the block's norm: the four lane groups add their partial sums in one
            //    order (each addition is commutative, so all four lanes agree)
            const float ssl = acc[0] + acc[1];
            const float a = ssl + __shfl_xor(ssl, 16, 64);
            const float nn = __builtin_sqrtf(a + __shfl_xor(a, 32, 64));
            nrm[c] = nn;

            // 4. butterflies over g', decision, packing, staging.  Everything runs in
            //    round-to-nearest except the last FMA of each decision, which adds 2^23
            //    under round-toward-minus-infinity (see round_down_fma4).
            const float rn = nn > 0.0f ? __builtin_amdgcn_rcpf(nn) : 0.0f;
            const float k1 = cb.g1 * rn, k2 = cb.g2 * rn * rn, k3 = cb.g3 * rn * rn * rn;
            const float hi = cb.clamp_t * nn, lo = -hi;
            uint32_t fb[4][8];                           // [g][position 8 G + i]: 2^23 + code
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = D[0][r][j], v1 = D[1][r][j], v2 = D[2][r][j], v3 = D[3][r][j];
                    const float a0 = v0 + v1, a1 = v0 - v1, a2 = v2 + v3, a3 = v2 - v3;
                    const float u[4] = {a0 + a2, a1 + a3, a0 - a2, a1 - a3};
                    float uc[4], pp[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        uc[g] = __builtin_amdgcn_fmed3f(u[g], lo, hi);
                        if constexpr (BITS == 3) {
                            pp[g] = __builtin_fmaf(__builtin_fabsf(uc[g]), k3, k2);
                            pp[g] = __builtin_fmaf(__builtin_fabsf(uc[g]), pp[g], k1);
                        } else {
                            pp[g] = k1;
                        }
                    }
                    float F[4];
                    round_down_fma4<(1 << (BITS - 1))>(uc, pp, F);
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        fb[g][4 * r + j] = __builtin_bit_cast(uint32_t, F[g]);
                }
            uint8_t *sb = stage + (16u * c + n) * CB;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t run = fb[g][7];
#pragma unroll
                for (int i = 6; i >= 0; --i)
                    run = lshl_add<BITS>(run, fb[g][i]);
                if constexpr (BITS == 3) {   // 24 bits at byte 12 g + 3 G
                    uint8_t *d = sb + 12 * g + 3u * G;
                    d[0] = (uint8_t)run;
                    d[1] = (uint8_t)(run >> 8);
                    d[2] = (uint8_t)(run >> 16);
                } else {                     // 16 bits at byte 8 g + 2 G
                    *(uint16_t *)(sb + 8 * g + 2u * G) = (uint16_t)run;
                }
            }
        }
        pb0 = b0;
        pnb = nb;
        // store_enc_tile writes block (lane & 31)'s norm from this lane
        pn16 = __builtin_bit_cast(uint16_t, (_Float16)__builtin_fminf((G & 1u) ? nrm[1] : nrm[0], 65504.0f));
        wave_lds_sync();   // staged codes visible
        tile = next;
        if (tile >= ntiles)
            break;
    }
    store_enc_tile<BITS>(stage, lane, pb0, pnb, pn16, row_blocks, cache_row_blocks, t0_blocks,
                         codes, norms);
}

// ---------------------------------------------------------------- decode
//
// x_hat = (n16 / 128) H y with H = H4 (x) H32 over p = 32 g + q, as in the encoder:
// v_g'[q] = sum_q' H32[q][q'] y[32 g' + q'] on v_mfma_f32_16x16x32_f16, then two
// butterfly stages over g' in registers with the rescale folded into the second.
// The levels enter as fp16 parts yh = fp16(y), yl = fp16(y - yh), two products each:
// yh + yl carries y to about 2^-22, the +-1 products are exact and the sums fp32.
//
// A wave takes 32 blocks as two 16-block column tiles; lane (G = lane / 16, n) takes
// block 16 c + n.  Its B operand for g' holds the levels of positions 32 g' + 8 G ..
// + 7: eight codes, one 24 / 16-bit field of the packed block (bytes 12 g' + 3 G /
// 8 g' + 2 G), as four lookups of two-code (yh pair, yl pair) entries.  After the
// butterflies it holds positions 32 g + 8 G .. + 7 for g = 0..3: four 16-byte stores.
// The codes arrive as whole 16-byte chunks (one instruction reads 16 blocks) through
// a small LDS stage per wave.  The grid gives every wave one tile.
template <int BITS, bool ROT>
__global__ __launch_bounds__(256, 4) void decode_kernel(const uint8_t *__restrict__ codes,
                                                            const uint16_t *__restrict__ norms,
                                                            uint32_t nblocks, uint32_t row_blocks,
                                                            int64_t cache_row_blocks,
                                                            int64_t t0_blocks,
                                                            uint8_t *__restrict__ x, Codebook cb,
                                                            Signs sg)
{
    constexpr int FB = 2 * BITS;   // index bits of a two-code entry
    constexpr int NE = 1 << FB;
    constexpr int CB = 16 * BITS;  // code bytes per block
    // entry e (first code in the low bits) -> (yh0 | yh1 << 16, yl0 | yl1 << 16),
    // kLdsCopies8 copies: copy c of entry e at (32 e + c) * 8, lane l reads copy l % 32
    __shared__ __attribute__((aligned(16))) uint8_t table[NE * kLdsCopies8 * 8];
    // per wave: the tile's codes, then (once every field is in registers) one column
    // tile's fp16 output at a time, block b at b * 256 with 16-byte chunk k at
    // (k ^ b) * 16
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWavesPerGroup][16 * kBlock * 2];
    static_assert(kEncTileBlocks * CB <= 16 * kBlock * 2, "the codes fit the output stage");
    __shared__ float lv[8];
    __shared__ uint2 ent_s[NE];
    // randomised rotation: the sign masks of a block's 16 chunks, built once per
    // workgroup (a wave has a single tile, so building them per lane would cost it
    // about a sixth of its VALU work)
    __shared__ u4_t smask_s[ROT ? 16 : 1];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n = lane & 15u, G = lane >> 4;
    const uint32_t ntiles = (nblocks + kEncTileBlocks - 1) / kEncTileBlocks;
    // cache position of block b: b itself when the cache rows hold exactly the
    // decoded rows (no division)
    const bool contig = cache_row_blocks == (int64_t)row_blocks && t0_blocks == 0;
    auto src_of = [&](uint32_t b) -> int64_t {
        if (contig)
            return (int64_t)b;
        return cache_block(b, row_blocks, cache_row_blocks, t0_blocks);
    };
    const uint32_t stride = gridDim.x * kWavesPerGroup;
    uint32_t tile = blockIdx.x * kWavesPerGroup + wave;
    // loads of tile t: lane (G, n), G < BITS, takes 16-byte chunk G of block 16 c + n
    // (one instruction covers 16 whole blocks, contiguous when the cache is); lanes
    // G >= BITS repeat chunk BITS - 1 (same addresses) and lanes past the tile's blocks
    // read its last block, so every load is unconditional
    u4_t C[2];
    uint16_t N16[2];
    auto load_tile = [&](uint32_t t) {
        const uint32_t tb0 = t * kEncTileBlocks;
        const uint32_t tnb = min(nblocks - tb0, (uint32_t)kEncTileBlocks);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int64_t src = src_of(tb0 + min(16u * c + n, tnb - 1u));
            C[c] = ld_stream((const u4_t *)(codes + src * CB) + min(G, (uint32_t)BITS - 1u));
            N16[c] = ld_stream(norms + src);
        }
    };
    // turbo3: the first tile's loads go out before the table set-up and its barriers
    // (3-5 % on whole caches); turbo2, whose table is a quarter the size, measured 1-3 %
    // slower that way and loads at the top of the loop
    constexpr bool kEarly = BITS == 3;
    if (kEarly && tile < ntiles)
        load_tile(tile);
    levels_to_lds(lv, cb);
    if constexpr (ROT) {
        if (threadIdx.x >= 64u && threadIdx.x < 80u)
            smask_s[threadIdx.x - 64u] = sign_mask_chunk(sg, threadIdx.x - 64u);
    }
    __syncthreads();
    // each entry is converted once (thread e), then copied: consecutive lanes write
    // consecutive copies, which meets every bank once
    if (threadIdx.x < (uint32_t)NE) {
        const uint32_t e = threadIdx.x;
        _Float16 a0, c0, a1, c1;
        split_f16(lv[e & ((1u << BITS) - 1u)], a0, c0);
        split_f16(lv[e >> BITS], a1, c1);
        ent_s[e] = uint2{pack_h2(a0, a1), pack_h2(c0, c1)};
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < (uint32_t)(NE * kLdsCopies8); i += kGroupThreads)
        *(uint2 *)(table + i * 8) = ent_s[i / kLdsCopies8];
    __syncthreads();

    if (tile >= ntiles)
        return;

    // A operands, as in the encoder: row tile r, lane row n -> H32 row
    // q = 8 (n / 4) + 4 r + n % 4, k-slots 8 G + s: (-1)^popcount(q & k) as fp16
    h8_t A[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint32_t q = 8u * (n >> 2) + 4u * r + (n & 3u);
        uint32_t w[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const uint32_t k0 = 8u * G + 2u * s2;
            const uint32_t h0 = (__builtin_popcount(q & k0) & 1u) ? 0xBC00u : 0x3C00u;
            const uint32_t h1 = (__builtin_popcount(q & (k0 + 1u)) & 1u) ? 0xBC00u : 0x3C00u;
            w[s2] = h0 | (h1 << 16);
        }
        A[r] = __builtin_bit_cast(h8_t, u4_t{w[0], w[1], w[2], w[3]});
    }
    // randomised rotation: the lane's output chunk g is chunk 4 g + G of its block
    u4_t smask[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        smask[g] = ROT ? smask_s[4u * g + G] : u4_t{0, 0, 0, 0};
    const uint32_t tcopy = (uint32_t)(uintptr_t)(lds_u8 *)table + (lane % kLdsCopies8) * 8;
    // the wave's codes stage: block 16 c + n of the tile at (16 c + n) * 16 BITS
    uint8_t *stage = stage_all[wave];
    // turbo3: the field of g' starts at byte 12 g' + 3 G = dword 3 g' + (3 G) / 4,
    // bit 8 ((3 G) % 4); it spills into the next dword only for G = 1, 2 (lane groups
    // 0 and 3 read their one dword twice, which keeps G = 3, g' = 3 inside the block)
    const uint32_t fdw = (3u * G) >> 2, fsh = 8u * ((3u * G) & 3u), fhi = fsh > 8u ? 1u : 0u;

    for (;;) {
        const uint32_t b0 = tile * kEncTileBlocks;
        const uint32_t nb = min(nblocks - b0, (uint32_t)kEncTileBlocks);
        if (!kEarly)
            load_tile(tile);
        wave_lds_sync();   // the previous tile's stage reads are done
#pragma unroll
        for (int c = 0; c < 2; ++c)
            if (G < (uint32_t)BITS)
                *(u4_t *)(stage + (16u * c + n) * CB + 16u * G) = C[c];
        wave_lds_sync();
        uint32_t F[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint8_t *blk = stage + (16u * c + n) * CB;
#pragma unroll
            for (int gp = 0; gp < 4; ++gp) {
                if constexpr (BITS == 3) {
                    const uint32_t *p = (const uint32_t *)blk + 3 * gp + fdw;
                    F[c][gp] = __builtin_amdgcn_alignbit(p[fhi], p[0], fsh);
                } else {
                    F[c][gp] = ((const uint16_t *)blk)[4 * gp + G];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f4_t D[4][2];
#pragma unroll
            for (int gp = 0; gp < 4; ++gp) {
                uint32_t bh[4], bl[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t e = __builtin_amdgcn_ubfe(F[c][gp], FB * j, FB);
                    const uint64_t t = lds_load<uint64_t>(lshl_add<8>(e, tcopy));
                    bh[j] = (uint32_t)t;
                    bl[j] = (uint32_t)(t >> 32);
                }
                const h8_t Bh = __builtin_bit_cast(h8_t, u4_t{bh[0], bh[1], bh[2], bh[3]});
                const h8_t Bl = __builtin_bit_cast(h8_t, u4_t{bl[0], bl[1], bl[2], bl[3]});
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    D[gp][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A[r], Bh, f4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    D[gp][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r], Bl, D[gp][r], 0, 0, 0);
                }
            }
            // u[32 g + 8 G + 4 r + j] = (n16 / 128) sum_g' H4[g][g'] D[g'][r][j]
            const float s = (float)__builtin_bit_cast(_Float16, N16[c]) * (1.0f / 128.0f);
            float u[4][8];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = D[0][r][j], v1 = D[1][r][j], v2 = D[2][r][j], v3 = D[3][r][j];
                    const float a0 = v0 + v1, a1 = v0 - v1, a2 = v2 + v3, a3 = v2 - v3;
                    const float as0 = a0 * s, as1 = a1 * s;
                    u[0][4 * r + j] = __builtin_fmaf(a2, s, as0);
                    u[1][4 * r + j] = __builtin_fmaf(a3, s, as1);
                    u[2][4 * r + j] = __builtin_fmaf(-a2, s, as0);
                    u[3][4 * r + j] = __builtin_fmaf(-a3, s, as1);
                }
            // every lane's fields (c = 0) or the previous column tile's rows (c = 1)
            // have been read: the stage takes this column tile's output
            wave_lds_sync();
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    h2_t hv = {(_Float16)u[g][2 * k], (_Float16)u[g][2 * k + 1]};
                    o[k] = __builtin_bit_cast(uint32_t, hv);
                }
                const u4_t ov = u4_t{o[0], o[1], o[2], o[3]};
                *(u4_t *)(stage + swz(n, 4u * g + G)) = ROT ? ov ^ smask[g] : ov;
            }
            // the column tile leaves as 1 KB-contiguous stores: lane l writes chunk
            // l % 16 of its block 4 k + l / 16
            wave_lds_sync();
            uint8_t *dst = x + (size_t)(b0 + 16u * c) * (kBlock * 2) + lane * 16u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t blk = 4u * k + (lane >> 4);
                const u4_t r = *(const u4_t *)(stage + swz(blk, lane & 15u));
                if (16u * c + blk < nb)
                    *(u4_t *)(dst + k * 1024) = r;
            }
        }
        tile += stride;
        if (tile >= ntiles)
            break;
        if (kEarly)
            load_tile(tile);   // (a capped grid) the next tile's loads
    }
}

// ---------------------------------------------------------------- q.K scores
//
// scores[h, t] = scale * sum_j (n16[t, j] / 128) * (H q_j[h]) . y[t, j], y the
// looked-up levels of key block j of cache row t.  Per kv head this is a
// [query heads x 128] by [128 x tokens] contraction for every block j, done on the
// matrix cores with v_mfma_f32_16x16x32_f16 (16 rows x 16 token columns, 32
// products per row and column).
//
// Precision.  Operands are fp16, accumulation is float.  Each rotated query value
// x is split into hi = fp16(x) and lo = fp16(x - hi), each codebook level y into
// yh = fp16(y) and yl = fp16(y - yh).  Rows 0..7 of A carry the hi parts of up to
// eight query heads, rows 8..15 their lo parts, and every value takes two products
// of its column: x * yh and x * yl.  Row h plus row 8 + h is then
// (hi + lo) . (yh + yl), x . y to about 2^-22 relative per term, plus float
// accumulation.  x is the rotated query times scale / 128 times a power of two that
// brings the head's largest |x| into [2^13, 2^14): no fp16 overflow and full fp16
// precision for queries of any magnitude; the power is divided out at the end.
//
// Operand layout (the instruction's lanes: lane l holds row l % 16 of A and column
// l % 16 of B, the same eight products 8 (l / 16) .. + 7 of both, and rows
// 4 (l / 16) .. + 3 of column l % 16 of the result).  Lane l scores token l % 16
// of a 16-token group; lane group p = l / 16 covers values [32 p, 32 p + 32) of
// each 128-block, whose 32 codes are one 12-byte (turbo3) / 8-byte (turbo2) run of
// the packed block.  Chunk c (0..7) of the run is values v0..v3 = 32 p + 4 c + 0..3
// and fills the eight products as
//   B: yh(v0) yh(v1) yl(v0) yl(v1) yh(v2) yh(v3) yl(v2) yl(v3)
//   A:  x(v0)  x(v1)  x(v0)  x(v1)  x(v2)  x(v3)  x(v2)  x(v3)
// so B is two 8-byte (hi pair, lo pair) entries of a two-value LDS table indexed by
// 6 code bits for turbo3, one 16-byte entry of a four-value table indexed by 8 code
// bits for turbo2.


// (group, block) units whose codes are in flight while the previous ones are
// scored; a group is the 16 tokens one wave scores at once.
constexpr int kQkDepth = 4;
constexpr int kQkHeads = 8;         // query heads per pass
constexpr int kQkGroupsPerCu = 4;   // workgroups per CU the grid aims at (4 waves per SIMD)
// turbo3 with one block per row fits a fifth group (92 VGPRs, 20 KB of LDS); turbo2's
// 36 KB of LDS allows four; with two blocks per row the query operands of both stay in
// registers: 3 groups per CU
constexpr int qk_groups_per_cu(int bits, int64_t m)
{
    return m == 2 ? 3 : bits == 3 && m == 1 ? 5 : kQkGroupsPerCu;
}
// turbo3: 64 two-value entries of 8 B, kLdsCopies8 copies (conflict-free);
// turbo2: 256 four-value entries of 16 B, 8 copies (16 B lookups are served 16 lanes
// per cycle, so lanes l and l + 8 may meet: the full 16 copies would take 64 KB and
// halve the workgroups per CU, which costs more than the conflicts).
constexpr int qk_table_bytes(int bits) { return bits == 3 ? 64 * kLdsCopies8 * 8 : 256 * 8 * 16; }
// LDS of a workgroup: table | query operands [m][16 rows][128] fp16 | 8 floats
inline size_t qk_smem_bytes(int bits, int64_t m)
{
    return (size_t)qk_table_bytes(bits) + (size_t)m * 16 * kBlock * 2 + kQkHeads * 4;
}



// x as packed fp16 (hi, lo): hi = fp16(x), lo = fp16(x - hi), both rounded to nearest
// even.  Two instructions: the conversion writes hi into the low half, and a mixed-
// precision FMA takes hi back as an fp16 operand, forms x - hi exactly in fp32 and
// writes its fp16 rounding into the high half (the compiler's own form takes four).
__device__ __forceinline__ uint32_t split_pack(float x)
{
    uint32_t d;
    asm("v_cvt_f16_f32 %0, %1\n\tv_fma_mixhi_f16 %0, -%0, 1.0, %1 op_sel_hi:[1,0,0]"
        : "=&v"(d) : "v"(x));
    return d;
}


// The q.K table (two-value entries for turbo3, four-value for turbo2): entry e,
// copy c at (e * NC + c) * EB; lane l reads copy l % NC.
template <int BITS>
struct QkTable {
    static constexpr int NE = BITS == 3 ? 64 : 256;           // entries (two / four codes)
    static constexpr int EB = BITS == 3 ? 8 : 16;             // bytes per entry
    static constexpr int NC = BITS == 3 ? kLdsCopies8 : 8;    // copies
    static constexpr int ES = BITS == 3 ? 8 : 7;              // log2 of the entry stride NC * EB
    static_assert(NC * EB == (1 << ES), "entry stride");
    static_assert(NE * NC * EB == qk_table_bytes(BITS), "table size");
};

// Fills the table of (yh, yl) pairs in the B order: entry e holds the values of codes
// e & 7, e >> 3 (turbo3) or (e >> 2 k) & 3, k = 0..3 (turbo2).  Whole workgroup; lv
// are the levels, already in LDS.  Each entry is converted once, into `scratch` (NE *
// EB bytes of LDS the caller does not use until after this call), then copied with
// consecutive lanes writing consecutive copies; ends with a barrier.
template <int BITS>
__device__ __forceinline__ void qk_fill_table(uint8_t *table, const float *lv, uint8_t *scratch)
{
    using Tb = QkTable<BITS>;
    static_assert(Tb::NE * Tb::EB <= 16 * kBlock * 2, "the entries fit one block's query operands");
    for (uint32_t e = threadIdx.x; e < (uint32_t)Tb::NE; e += kGroupThreads) {
        if constexpr (BITS == 3) {
            _Float16 a0, a1, c0, c1;
            split_f16(lv[e & 7], a0, c0);
            split_f16(lv[e >> 3], a1, c1);
            *(uint2 *)(scratch + e * Tb::EB) = uint2{pack_h2(a0, a1), pack_h2(c0, c1)};
        } else {
            _Float16 a[4], c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                split_f16(lv[(e >> (2 * k)) & 3], a[k], c[k]);
            *(uint4 *)(scratch + e * Tb::EB) = uint4{pack_h2(a[0], a[1]), pack_h2(c[0], c[1]),
                                                      pack_h2(a[2], a[3]), pack_h2(c[2], c[3])};
        }
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < (uint32_t)(Tb::NE * Tb::NC); i += kGroupThreads) {
        if constexpr (BITS == 3)
            *(uint2 *)(table + i * Tb::EB) = *(const uint2 *)(scratch + (i / Tb::NC) * Tb::EB);
        else
            *(uint4 *)(table + i * Tb::EB) = *(const uint4 *)(scratch + (i / Tb::NC) * Tb::EB);
    }
    __syncthreads();
}


// Query operands.  Wave w prepares heads w and w + 4 of the pass (h0 .. h0 + nh - 1):
// rotates every 128-slice (lane l holds positions l and 64 + l; span 64 in-lane, spans
// 32..1 across lanes), takes the head's largest |q'|, then writes x = q' * scale / 128 *
// 2^(14 - e) as hi (row hh) and lo (row 8 + hh) of qa [m][16][128], and 2^(e - 14) to
// pw_s[hh].  Heads past nh get zero rows.  The caller barriers afterwards.  With the
// randomised rotation q' = H D q, since q . (D H y) = (H D q) . y.
// The query values lane `lane` of wave `wave` rotates when D == 128 (positions lane and
// 64 + lane of its two heads' rows), loaded at the very start of a kernel: issued before
// the first key codes, they do not wait behind them (loads complete in order).  Heads
// past nh read head h0's row instead (never used).
__device__ __forceinline__ void qk_load_queries(uint16_t (&pre)[2][2], const uint16_t *__restrict__ q,
                                                uint32_t b, uint32_t Hq, uint32_t h0, uint32_t nh,
                                                uint32_t wave, uint32_t lane)
{
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t hh = wave + kWavesPerGroup * s;
        const uint16_t *qv = q + ((size_t)b * Hq + h0 + (hh < nh ? hh : 0u)) * kBlock;
        pre[s][0] = ld_stream(qv + lane);
        pre[s][1] = ld_stream(qv + 64 + lane);
    }
}

template <bool ONE_BLOCK>
__device__ __forceinline__ void qk_prepare_queries(_Float16 *qa, float *pw_s,
                                                   const uint16_t *__restrict__ q, uint32_t b,
                                                   uint32_t Hq, uint32_t h0, uint32_t nh,
                                                   uint32_t m, uint32_t wave, uint32_t lane,
                                                   float scale, const Signs &sg,
                                                   const uint16_t (&pre)[2][2])
{
    const uint16_t fa = (uint16_t)(sign_mask_f32(sg, lane) >> 16);
    const uint16_t fc = (uint16_t)(sign_mask_f32(sg, 64u + lane) >> 16);
    // the slice's two values (from memory, or preloaded by qk_load_queries: D == 128)
    auto rotate_v = [&](uint16_t va, uint16_t vc, float &a, float &c) {
        a = (float)__builtin_bit_cast(_Float16, (uint16_t)(va ^ fa));
        c = (float)__builtin_bit_cast(_Float16, (uint16_t)(vc ^ fc));
        const float s0 = a + c;
        c = a - c;
        a = s0;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {
            const float pa = __shfl_xor(a, h, 64), pc = __shfl_xor(c, h, 64);
            const bool up = (lane & (uint32_t)h) != 0u;
            a = up ? pa - a : a + pa;
            c = up ? pc - c : c + pc;
        }
    };
    auto rotate = [&](const uint16_t *v, float &a, float &c) { rotate_v(v[lane], v[64 + lane], a, c); };
    static_assert(kQkHeads == 2 * kWavesPerGroup, "two preloaded head slots per wave");
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
        const uint32_t hh = wave + kWavesPerGroup * slot;
        _Float16 *hi_row = qa + hh * kBlock, *lo_row = qa + (kQkHeads + hh) * kBlock;
        if (hh < nh) {
            const uint16_t *qv = q + ((size_t)b * Hq + h0 + hh) * ((size_t)m * kBlock);
            float mx = 0.0f, a1 = 0.0f, c1 = 0.0f;   // a1, c1: the single slice when m == 1
            for (uint32_t j = 0; j < m; ++j) {
                float a, c;
                if (ONE_BLOCK)
                    rotate_v(pre[slot][0], pre[slot][1], a, c);
                else
                    rotate(qv + j * kBlock, a, c);
                mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(c)));
                a1 = a;
                c1 = c;
            }
#pragma unroll
            for (int h = 32; h >= 1; h >>= 1)
                mx = __builtin_fmaxf(mx, __shfl_xor(mx, h, 64));
            int e = 0;
            (void)frexpf(mx * __builtin_fabsf(scale) * (1.0f / 128.0f), &e);
            const float f = ldexpf(scale * (1.0f / 128.0f), 14 - e);
            for (uint32_t j = 0; j < m; ++j) {
                float a = a1, c = c1;
                if (!ONE_BLOCK)
                    rotate(qv + j * kBlock, a, c);
                _Float16 ah, al, ch, cl;
                split_f16(a * f, ah, al);
                split_f16(c * f, ch, cl);
                hi_row[j * 2048 + lane] = ah;
                hi_row[j * 2048 + 64 + lane] = ch;
                lo_row[j * 2048 + lane] = al;
                lo_row[j * 2048 + 64 + lane] = cl;
            }
            if (lane == 0)
                pw_s[hh] = ldexpf(1.0f, e - 14);
        } else {
            for (uint32_t j = 0; j < m; ++j) {
                hi_row[j * 2048 + lane] = hi_row[j * 2048 + 64 + lane] = (_Float16)0.0f;
                lo_row[j * 2048 + lane] = lo_row[j * 2048 + 64 + lane] = (_Float16)0.0f;
            }
            if (lane == 0)
                pw_s[hh] = 0.0f;
        }
    }
}

// One 16-row unit of q.K: the eight 16 x 16 x 32 products of the query operands A
// (row lane % 16, values of the lane's run) with the lane's 32 key codes w (row
// lane % 16, run lane / 16), looked up in this lane's table copy tcopy.  Result rows
// 4 (lane / 16) .. + 3 of column lane % 16, not yet scaled by the norm.
template <int BITS>
__device__ __forceinline__ f4_t qk_unit(const h8_t (&A)[8], const uint32_t *w, uint32_t tcopy)
{
    constexpr int ES = QkTable<BITS>::ES;
    // two accumulation chains (even / odd chunks) halve the dependent MFMA latency
    f4_t D[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u4_t bv;
        if constexpr (BITS == 3) {
            uint32_t o[2];   // LDS addresses of the entries of v0 v1 and v2 v3
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int bit = 12 * c + 6 * k2, wi = bit >> 5, sh = bit & 31;
                const uint32_t e = sh <= 26 ? __builtin_amdgcn_ubfe(w[wi], sh, 6)
                                            : __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 63u;
                o[k2] = lshl_add<ES>(e, tcopy);   // e * NC * EB + copy
            }
            const uint64_t r0 = lds_load<uint64_t>(o[0]), r1 = lds_load<uint64_t>(o[1]);
            bv = u4_t{(uint32_t)r0, (uint32_t)(r0 >> 32), (uint32_t)r1, (uint32_t)(r1 >> 32)};
        } else {
            const uint32_t e = __builtin_amdgcn_ubfe(w[c >> 2], 8 * (c & 3), 8);
            bv = lds_load<u4_t>(lshl_add<ES>(e, tcopy));
        }
        D[c & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[c], __builtin_bit_cast(h8_t, bv),
                                                          D[c & 1], 0, 0, 0);
    }
    return D[0] + D[1];
}

// BITS: 2 or 3.  MF: blocks per row of the batched path (1: D == 128, 2: D == 256; the
// query operands of every block stay in registers), or 0: the general path for D = 128 m,
// m >= 3 (query operands read from LDS per unit, per-unit norm loads and per-lane score
// stores).  A
// workgroup scores cache rows [blockIdx.y * tpg, +tpg) of one (sequence, kv head) for up
// to eight query heads (pass blockIdx.x % passes).
template <int BITS, int MF>
__global__ __launch_bounds__(256, qk_groups_per_cu(BITS, MF)) void qk_kernel(const uint8_t *__restrict__ k_codes,
                                                    const uint16_t *__restrict__ k_norms,
                                                    const uint16_t *__restrict__ q,
                                                    float *__restrict__ scores, uint32_t Hkv,
                                                    int64_t Tc, uint32_t T, uint32_t m_arg,
                                                    uint32_t G, uint32_t Hq, uint32_t passes,
                                                    uint32_t tpg, float scale, Codebook cb,
                                                    Signs sg)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t qk_smem[];
    constexpr bool FAST = MF > 0;              // the batched path
    constexpr uint32_t MD = FAST ? MF : 1;     // (a divisor for the batched path's arithmetic)
    constexpr int NC = QkTable<BITS>::NC;
    constexpr int EB = QkTable<BITS>::EB;
    constexpr int CB = 16 * BITS;              // code bytes per block
    constexpr int LW = BITS;                   // code words per lane (32 codes)
    const uint32_t m = FAST ? MD : m_arg;      // blocks per row
    uint8_t *table = qk_smem;
    _Float16 *qa = (_Float16 *)(qk_smem + qk_table_bytes(BITS));   // [m][16][128]
    float *pw_s = (float *)(qk_smem + qk_table_bytes(BITS) + (size_t)m * 16 * kBlock * 2);

    const uint32_t pass = blockIdx.x % passes;
    const uint32_t bg = blockIdx.x / passes;           // b * Hkv + g
    const uint32_t b = bg / Hkv, g = bg - b * Hkv;
    const uint32_t h0 = g * G + pass * kQkHeads;       // first query head of this pass
    const uint32_t nh = min(G - pass * kQkHeads, (uint32_t)kQkHeads);

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar
    const uint32_t n = lane & 15u, part = lane >> 4;
    const uint32_t t_begin = blockIdx.y * tpg;
    const uint32_t t_end = min(T, t_begin + tpg);
    const size_t row0 = (size_t)bg * Tc;               // first cache row of (b, g)

    // This wave's units: the wave owns the contiguous rows [first, last) of the
    // chunk; unit k is block k % m of group k / m, and group i covers rows
    // first + 16 i + [0, 16).  Contiguous rows keep each wave's reads, norm lines and
    // score lines to itself.
    const uint32_t wspan = tpg / kWavesPerGroup;
    const uint32_t first = t_begin + wave * wspan;
    const uint32_t last = min(t_end, first + wspan);
    const uint32_t ngroups = first < last ? (last - first + 15u) / 16u : 0u;
    const uint32_t nunits = ngroups * m;

    // Codes (and, on the general path, the norm) of this lane's run of unit k.  Loads
    // are unconditional, so the prefetch is straight-line code: rows past the wave's
    // range are clamped to its last row (a wave without rows: the chunk's last), so they
    // re-read lines the wave has just fetched instead of the next wave's rows, which
    // would come from HBM a second time; their values are never stored.  The group's
    // base address is wave-uniform (scalar) and each lane adds a 32-bit offset.
    const uint32_t row_bytes = m * CB;
    const uint32_t lastc = first < last ? last - 1u : t_end - 1u;
    auto fetch = [&](uint32_t k, uint32_t (&w)[LW], uint16_t &nr) {
        const uint32_t gi = FAST ? k / MD : k / m;
        const uint32_t j = k - gi * m;
        const uint32_t tb = min(first + gi * 16u, lastc);
        const uint32_t r = min(n, lastc - tb);
        const size_t blk0 = (row0 + tb) * m + j;
        const uint32_t *src =
            (const uint32_t *)(k_codes + blk0 * CB + (__umul24(r, row_bytes) + part * (4 * BITS)));
#pragma unroll
        for (int i = 0; i < LW; ++i)
            w[i] = ld_stream(src + i);
        if constexpr (!FAST)
            nr = ld_stream(k_norms + blk0 + __umul24(r, m));
    };
    // Batched path: a batch of kQkDepth units holds 64 (row, block) pairs, whose norms
    // come in one load (element e0 + lane from the batch's first row, clamped to the
    // last element of the wave's last row, as the codes); each unit takes its pair's
    // norm from the lane that holds it.  A separate small load per unit would cost the
    // memory pipeline about as much as the unit's codes.
    static_assert(kQkDepth * 16 == 64, "one norm load per batch");
    auto fetch_norms = [&](uint32_t k, uint16_t &na) {
        const size_t e0 = (row0 + first + 16u * (k / MD)) * MD;
        const size_t emax = (row0 + lastc) * MD + (MD - 1u);
        na = ld_stream(k_norms + min(e0 + lane, emax));
    };
    uint16_t qpre[2][2] = {{0, 0}, {0, 0}};
    if constexpr (MF == 1)   // the queries first: their wait does not cover the codes
        qk_load_queries(qpre, q, b, Hq, h0, nh, wave, lane);
    uint32_t wn[kQkDepth][LW];
    uint16_t nn[kQkDepth];
    // (16-bit, widened only where used: a widening right after the load would wait
    // for it there)
    uint16_t nna = 0;
#pragma unroll
    for (int d = 0; d < kQkDepth; ++d)
        fetch(d, wn[d], nn[d]);
    if constexpr (FAST)
        fetch_norms(0, nna);

    __shared__ float lv[8];
    levels_to_lds(lv, cb);
    __syncthreads();
    qk_fill_table<BITS>(table, lv, (uint8_t *)qa);   // qa is written only below

    qk_prepare_queries<MF == 1>(qa, pw_s, q, b, Hq, h0, nh, m, wave, lane, scale, sg, qpre);
    __syncthreads();

    // A operands of block j for this lane's row (lane % 16) and value run
    const _Float16 *arow = qa + n * kBlock + part * 32;
    auto load_a = [&](uint32_t j, h8_t (&A)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t *p = (const uint32_t *)(arow + j * 2048 + 4 * c);
            const uint32_t x01 = p[0], x23 = p[1];
            A[c] = __builtin_bit_cast(h8_t, u4_t{x01, x01, x23, x23});
        }
    };
    h8_t A[MD][8];
    if constexpr (FAST) {
#pragma unroll
        for (int j = 0; j < (int)MD; ++j)
            load_a(j, A[j]);
        __syncthreads();   // every wave holds its operands: qa is free for the score stages
    }
    // LDS address of this lane's table copy (entries are addressed as integers so that
    // each lookup is one bit-field extract and one shift-add)
    const uint32_t tcopy = (uint32_t)(uintptr_t)(lds_u8 *)table + (lane % NC) * EB;
    // after the hi/lo combine, lane l holds query heads hu and hu + 2 of token l % 16
    const uint32_t hu = 4u * (part & 1u) + (lane >> 5);
    const float pw_u = pw_s[hu], pw_v = pw_s[hu + 2];
    float* const out_u = scores + ((size_t)b * Hq + h0 + hu) * T;
    float* const out_v = scores + ((size_t)b * Hq + h0 + hu + 2) * T;
    // Batched path: the scores of two row groups (32 rows x 8 heads) gather in a 1 KB
    // stage per wave (the query operands' LDS, free once they are in registers) and leave
    // as one store of 16 bytes per lane, a whole 128-byte line per head (lane l: head
    // l / 8, rows 4 (l % 8) .. + 3)
    float *stg = (float *)qa + wave * (kQkHeads * 32);
    const bool rows16 = (T & 3u) == 0u && ((uintptr_t)scores & 15u) == 0u;   // rows 16-byte aligned
    const uint32_t sh = lane >> 3, sr = 4u * (lane & 7u);
    float *const out_s = scores + ((size_t)b * Hq + h0 + sh) * T;
    // the source lane of the norm of (row group rg, block j) of a batch, and the score of
    // a finished row group into the stage
    auto batch_norm = [&](int rg, int j, uint16_t na) -> float {
        const int src = (16 * rg + (int)n) * (int)MD + j;
        const uint16_t nr16 = (uint16_t)__shfl((int)(uint32_t)na, src, 64);
        return (float)__builtin_bit_cast(_Float16, nr16);
    };

    f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t k0 = 0;
    if constexpr (FAST) {
        // Whole batches (64 / MF rows inside the wave's range, 16-byte aligned score
        // rows): the next batch's loads are unconditional (rows clamped inside the
        // chunk), every lane stores a 16-byte score line per pair of row groups (a lane
        // whose head is past the pass's last one writes that head's line again, with the
        // same values), and the next batch's codes are taken at the end of the batch.
        // The loop body then has no branch around a memory operation, and the wait for
        // the prefetched codes counts exactly the score stores issued after them.
        constexpr uint32_t RPB = 16 * kQkDepth / MD;   // rows per batch
        const uint32_t nfull = rows16 && first < last ? (last - first) / RPB * kQkDepth : 0u;
        const uint32_t shf = min(sh, nh - 1u);
        float *const out_f = scores + ((size_t)b * Hq + h0 + shf) * T;
        uint32_t wc[kQkDepth][LW];
        uint16_t nca = nna;
#pragma unroll
        for (int d = 0; d < kQkDepth; ++d)
#pragma unroll
            for (int i = 0; i < LW; ++i)
                wc[d][i] = wn[d][i];
        for (; k0 < nfull; k0 += kQkDepth) {
            prio_by_progress(k0, nfull);
#pragma unroll
            for (int d = 0; d < kQkDepth; ++d)
                fetch(k0 + kQkDepth + d, wn[d], nn[d]);
            fetch_norms(k0 + kQkDepth, nna);
#pragma unroll
            for (int d = 0; d < kQkDepth; ++d) {
                const int rg = d / (int)MD, jb = d % (int)MD;   // row group, block
                const f4_t Du = qk_unit<BITS>(A[jb], wc[d], tcopy) * batch_norm(rg, jb, nca);
                acc = jb == 0 ? Du : acc + Du;
                if (jb == (int)MD - 1) {
                    float s0 = acc[0], s1 = acc[1], s2 = acc[2], s3 = acc[3];
                    swap32(s0, s1);
                    swap32(s2, s3);
                    stg[hu * 32 + 16 * (rg & 1) + n] = (s0 + s1) * pw_u;
                    stg[(hu + 2) * 32 + 16 * (rg & 1) + n] = (s2 + s3) * pw_v;
                    if (rg & 1) {
                        wave_lds_sync();
                        const float4 sv = *(const float4 *)(stg + shf * 32 + sr);
                        *(float4 *)(out_f + first + (k0 / MD + rg - 1u) * 16u + sr) = sv;
                        wave_lds_sync();   // the stage is read before the next pair writes it
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < kQkDepth; ++d)
#pragma unroll
                for (int i = 0; i < LW; ++i)
                    wc[d][i] = wn[d][i];
            nca = nna;
        }
    }
    // Remaining units (all of them on the general path; at most one ragged batch on the
    // batched path, whose codes are already in wn).
    for (; k0 < nunits; k0 += kQkDepth) {
        uint32_t wc[kQkDepth][LW];
        uint16_t nc[kQkDepth];
#pragma unroll
        for (int d = 0; d < kQkDepth; ++d) {
#pragma unroll
            for (int i = 0; i < LW; ++i)
                wc[d][i] = wn[d][i];
            nc[d] = nn[d];
        }
        const uint16_t nca = nna;
        if (k0 + kQkDepth < nunits) {
#pragma unroll
            for (int d = 0; d < kQkDepth; ++d)
                fetch(k0 + kQkDepth + d, wn[d], nn[d]);
            if constexpr (FAST)
                fetch_norms(k0 + kQkDepth, nna);
        }
#pragma unroll
        for (int d = 0; d < kQkDepth; ++d) {
            const uint32_t k = k0 + d;
            if constexpr (FAST) {
                const int rg = d / (int)MD, jb = d % (int)MD;
                const uint32_t gi = k / MD;
                const f4_t Du = qk_unit<BITS>(A[jb], wc[d], tcopy) * batch_norm(rg, jb, nca);
                acc = jb == 0 ? Du : acc + Du;
                if (jb == (int)MD - 1) {
                    // rows h (hi) and 8 + h (lo) sit in lanes l and l + 32: one swap pairs them
                    float s0 = acc[0], s1 = acc[1], s2 = acc[2], s3 = acc[3];
                    swap32(s0, s1);
                    swap32(s2, s3);
                    stg[hu * 32 + 16 * (rg & 1) + n] = (s0 + s1) * pw_u;
                    stg[(hu + 2) * 32 + 16 * (rg & 1) + n] = (s2 + s3) * pw_v;
                    if (rg & 1) {
                        wave_lds_sync();
                        const float4 sv = *(const float4 *)(stg + sh * 32 + sr);
                        const uint32_t t = first + (gi - 1u) * 16u + sr;   // the pair's first row + sr
                        if (sh < nh) {
                            if (rows16 && t + 3u < last) {
                                *(float4 *)(out_s + t) = sv;
                            } else {
                                const float e[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (t + i < last)
                                        out_s[t + i] = e[i];
                            }
                        }
                        wave_lds_sync();   // the stage is read before the next pair writes it
                    }
                }
            } else {
                const uint32_t gi = k / m;
                const uint32_t j = k - gi * m;
                load_a(j, A[0]);
                const float nf = (float)__builtin_bit_cast(_Float16, nc[d]);
                acc += qk_unit<BITS>(A[0], wc[d], tcopy) * nf;
                if (j == m - 1u) {
                    float s0 = acc[0], s1 = acc[1], s2 = acc[2], s3 = acc[3];
                    swap32(s0, s1);
                    swap32(s2, s3);
                    const float u = (s0 + s1) * pw_u, v = (s2 + s3) * pw_v;
                    const uint32_t t = first + gi * 16u + n;
                    if (t < last) {
                        if (hu < nh)
                            out_u[t] = u;
                        if (hu + 2u < nh)
                            out_v[t] = v;
                    }
                    acc = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
    }
}

// ---------------------------------------------------------------- decode attention
//
// out[b, h, :] = sum_t p_t v_hat_t with p = softmax_t(scale q . k_hat_t) over cache rows
// [0, T): the fused read carried through softmax and the values.  Since
// v_hat_t = (n_t / 128) H y_t and H is linear,
//   sum_t p_t v_hat_t = H (sum_t p_t n_t y_t) / 128,
// so the values are summed in the rotated domain and transformed once per head.
//
// attn_partial_kernel: a workgroup takes one (sequence, kv head, <= 8 query heads) and
// a chunk of rows; each wave scores its own rows exactly as qk_kernel does, keeps an
// online softmax per head (running max m, running sum l of exp(s - m)) and accumulates
// acc = sum_t exp(s_t - m) n_t y_t; the four waves' states are merged in LDS and the
// workgroup writes one (m, l, acc) per head to the workspace.  attn_combine_kernel:
// one workgroup per (sequence, query head) merges the chunks, transforms acc once and
// divides by 128 l.  Scores, m and the workspace's m are kept in log2 units (the
// query scale carries log2 e), so every exponential is one v_exp_f32.
//
// P.V runs on the matrix cores too: v_mfma_f32_16x16x32_f16 over the 16 rows (tokens)
// of a unit, for a set of four query heads.  Row r = 8 hilo + 2 hh + e of A stands for
// head hh of the set, value-position parity e and the fp16 hi (hilo 0) or lo (1) part
// of the weight w_t = exp(s_t - m) n_t 2^(15 - E); k-slots 8 j .. 8 j + 7 (lane group j)
// are tokens 2 j and 2 j + 1 of an 8-token block, each as (yh of parity 0, yh of
// parity 1, yl of parity 0, yl of parity 1).  A holds w in the slots of its own parity
// and zeros in the others, so column P of the product is sum_t w_t y_t at position
// 2 P + e in row e: the two positions of a pair take one row each.  That B layout is
// exactly what a two-code q.K table entry (positions 2 P, 2 P + 1 of one token) holds,
// so two lookups (tokens 2 j, 2 j + 1) fill a B operand with no register moves.  Column n of
// product block c is pair 4 n + c: the lane of column n needs positions 8 n .. 8 n + 7
// of its four tokens, eight codes that are one contiguous 24-bit (turbo3) / 16-bit
// (turbo2) field of each token's packed block.  Each wave parks its 16 tokens'
// packed codes in a small LDS tile (a 16 BITS-byte row per token and block) and every lane reads
// its four fields from it and looks the code pairs up: 16 lookups and 8 products per
// unit for up to four heads, 16 products for eight.
// The weights are written to a small LDS tile, as packed (hi, lo) fp16 pairs, by the
// lanes that computed them (two (head, token) pairs each) and read back into the A
// layout by byte permutes.  The softmax runs once per
// batch of four units (64 rows): one running-max update, one sum and one wave
// barrier for the batch's tiles.  w = exp(s - m) n 2^(15 - E), with E the exponent of
// the largest value norm seen so far, lies below 2^15, inside fp16's range, and keeps
// the lo part a normal number down to weights 2^-18 of the largest: the weights that
// follow a dominant row (on a row of zeros, say) keep their relative precision.  A
// larger E rescales acc by a power of two, the way a larger score rescales it by
// exp(m_old - m_new).

// Workgroups per CU, also the target of the row chunking; NHS = sets of four query heads.
// head_dim 128: turbo3 (37 KB of LDS) runs four with one head set, within 128 VGPRs (a
// few values live only in the prologue and after the loop spill, one reload per batch),
// and three with two sets (153 VGPRs; at four they spill 22); turbo2 (53 KB) runs three.
// head_dim 256 runs two: the second block's query operands (32 VGPRs) and accumulators do
// not fit three groups' registers for turbo3, reading the operands from LDS at each use
// instead costs more than the third group gains (325 against 248 us at 16 x 8 x 32768
// rows), and turbo2's third group (168 VGPRs) measured no faster.
constexpr int attn_groups_per_cu(int bits, int NHS, int M)
{
    return M == 2 ? 2 : bits == 3 && NHS == 1 ? 4 : 3;
}
// M = blocks per row (head_dim 128 M).  A batch is 64 / M rows (4 / M 16-row units), so
// that one norm load per lane covers its 64 (row, block) norms and the units in flight
// hold the same bytes for both head dims.
constexpr int attn_depth(int M) { return 4 / M; }
constexpr int attn_rec(int M) { return 4 + kBlock * M; }   // workspace floats per partial: m, l, -, -, acc
constexpr int kAttnWExp = 15;          // the weights' power-of-two headroom below fp16's max
constexpr float kLog2e = 1.44269504088896340736f;

// 2^x by the hardware's v_exp_f32 (2^-inf = 0).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value lookups: entry e (two codes, the first in the low bits) -> the dwords
// (yh0 | yh1 << 16, yl0 | yl1 << 16), kLdsCopies8 copies: for turbo3 the q.K table
// itself, for turbo2 a table of its own (the q.K entries there hold four codes).
constexpr int attn_vtable_bytes(int bits) { return bits == 3 ? 0 : 16 * kLdsCopies8 * 8; }

// NHS: sets of four query heads per pass (1: up to four heads, 2: up to eight).
// M: 128-blocks per row (1 or 2); each row's score sums its blocks' dot products, each
// block has its own value norms, weights and P.V accumulators.
template <int BITS, int NHS, int M>
__global__ __launch_bounds__(256, attn_groups_per_cu(BITS, NHS, M)) void attn_partial_kernel(
    const uint8_t *__restrict__ k_codes, const uint16_t *__restrict__ k_norms,
    const uint8_t *__restrict__ v_codes, const uint16_t *__restrict__ v_norms,
    const uint16_t *__restrict__ q, float *__restrict__ work, uint32_t Hkv, int64_t Tc,
    uint32_t T, uint32_t G, uint32_t Hq, uint32_t passes, uint32_t tpg, uint32_t nparts,
    float scale, Codebook cb, Signs sg)
{
    constexpr int NC = QkTable<BITS>::NC, EB = QkTable<BITS>::EB;
    constexpr int CB = 16 * BITS;        // code bytes per block
    constexpr int LW = BITS;             // code words per lane and block (32 codes)
    constexpr int DEPTH = attn_depth(M); // units per batch
    constexpr int REC = attn_rec(M);
    constexpr int RW = 4 * BITS * M;     // words per token row of a code tile (16 BITS B per block)
    // LDS: the tables; per unit in flight the packed value codes of its 16 rows (one
    // spare dword read past the last field) and, per block, the weights [head][row] as
    // (hi, lo); after the last unit the same bytes hold the four waves' states
    constexpr int kTables = qk_table_bytes(BITS) + attn_vtable_bytes(BITS);
    constexpr int kRawWords = 16 * RW + 4;
    constexpr int kRawBytes = DEPTH * kWavesPerGroup * kRawWords * 4;
    constexpr int kPtBytes = DEPTH * M * kWavesPerGroup * kQkHeads * 16 * 4;
    constexpr int kMerge = kWavesPerGroup * kQkHeads * REC * 4;
    static_assert(kMerge <= kTables + kRawBytes + kPtBytes, "the merge reuses the tiles' bytes");
    static_assert(DEPTH * 16 * M == 64, "one norm load per lane per batch");
    __shared__ __attribute__((aligned(16))) uint8_t smem[kTables + kRawBytes + kPtBytes];
    __shared__ __attribute__((aligned(16))) float ftile[kWavesPerGroup][kQkHeads];
    __shared__ float pw_s[kQkHeads];
    __shared__ float lv[8];
    uint8_t *ktable = smem, *vtable = BITS == 3 ? smem : smem + qk_table_bytes(BITS);
    uint32_t *raw_base = (uint32_t *)(smem + kTables);
    uint32_t *pt_base = (uint32_t *)(smem + kTables + kRawBytes);
    // the query operands, in the code tiles' bytes until every wave holds them in registers
    static_assert(M * 16 * kBlock * 2 <= kRawBytes, "qa fits the code tiles");
    _Float16 *qa = (_Float16 *)raw_base;

    const uint32_t pass = blockIdx.x % passes;
    const uint32_t bg = blockIdx.x / passes;           // b * Hkv + g
    const uint32_t b = bg / Hkv, g = bg - b * Hkv;
    const uint32_t h0 = g * G + pass * kQkHeads;       // first query head of this pass
    const uint32_t nh = min(G - pass * kQkHeads, (uint32_t)kQkHeads);

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n = lane & 15u, part = lane >> 4;
    const uint32_t t_begin = blockIdx.y * tpg;
    const uint32_t t_end = min(T, t_begin + tpg);
    const size_t row0 = (size_t)bg * Tc;

    // this wave's rows [first, last); unit k covers rows first + 16 k + [0, 16)
    const uint32_t wspan = tpg / kWavesPerGroup;
    const uint32_t first = t_begin + wave * wspan;
    const uint32_t last = min(t_end, first + wspan);
    const uint32_t nunits = first < last ? (last - first + 15u) / 16u : 0u;

    // K and V codes of this lane's run (row n, values 32 part ..) of every block of unit
    // k, and a batch's norms (element (row, block) of the batch's 64 / M rows, one per
    // lane).  Rows past the wave's range are clamped to its last row (a wave without
    // rows: the chunk's last), so the loads are unconditional, stay in bounds and
    // re-read lines the wave has just fetched; their values are never used.
    const uint32_t lastc = nunits ? last - 1u : t_end - 1u;
    auto fetch = [&](uint32_t k, uint32_t (&wk)[M][LW], uint32_t (&wv)[M][LW]) {
        const uint32_t tb = min(first + k * 16u, lastc);                 // wave-uniform
        const uint32_t r = min(n, lastc - tb);
        const size_t ub = (row0 + tb) * (M * CB);                        // wave-uniform
#pragma unroll
        for (int jb = 0; jb < M; ++jb) {
            const uint32_t lo = __umul24(r, (uint32_t)(M * CB)) + jb * CB + part * (4 * BITS);
            const uint32_t *kp = (const uint32_t *)(k_codes + ub + lo);
            const uint32_t *vp = (const uint32_t *)(v_codes + ub + lo);
#pragma unroll
            for (int i = 0; i < LW; ++i) {
                wk[jb][i] = ld_stream(kp + i);
                wv[jb][i] = ld_stream(vp + i);
            }
        }
    };
    auto fetch_norms = [&](uint32_t k, uint32_t &nk, uint32_t &nv) {
        const uint32_t tb = min(first + 16u * k, lastc);                 // wave-uniform
        const uint32_t e = min(lane, (lastc - tb) * M + (M - 1));
        nk = ld_stream(k_norms + (row0 + tb) * M + e);
        nv = ld_stream(v_norms + (row0 + tb) * M + e);
    };
    // a batch's codes and norms; each unit's registers are refilled with the next
    // batch's unit as soon as they have been consumed
    uint16_t qpre[2][2] = {{0, 0}, {0, 0}};
    if constexpr (M == 1)   // the queries first: see qk_load_queries
        qk_load_queries(qpre, q, b, Hq, h0, nh, wave, lane);
    uint32_t wk[DEPTH][M][LW], wv[DEPTH][M][LW];
    uint32_t nkc = 0, nvc = 0;
    fetch_norms(0, nkc, nvc);   // norms next, as in the loop
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        fetch(d, wk[d], wv[d]);

    // tables and query operands
    levels_to_lds(lv, cb);
    __syncthreads();
    qk_fill_table<BITS>(ktable, lv, (uint8_t *)qa);   // qa is written only below
    if constexpr (BITS == 2) {
        for (uint32_t i = threadIdx.x; i < 16u * kLdsCopies8; i += kGroupThreads) {
            const uint32_t e = i / kLdsCopies8;
            _Float16 a0, c0, a1, c1;
            split_f16(lv[e & 3u], a0, c0);
            split_f16(lv[e >> 2], a1, c1);
            *(uint2 *)(vtable + i * 8) = uint2{pack_h2(a0, a1), pack_h2(c0, c1)};
        }
    }
    qk_prepare_queries<M == 1>(qa, pw_s, q, b, Hq, h0, nh, (uint32_t)M, wave, lane, scale, sg, qpre);
    __syncthreads();

    // query operands of block jb for this lane's row (lane % 16) and value run, kept in
    // registers
    auto load_a = [&](uint32_t jb, h8_t (&Aj)[8]) {
        const _Float16 *arow = qa + jb * 2048 + n * kBlock + part * 32;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t *p = (const uint32_t *)(arow + 4 * c);
            const uint32_t x01 = p[0], x23 = p[1];
            Aj[c] = __builtin_bit_cast(h8_t, u4_t{x01, x01, x23, x23});
        }
    };
    h8_t A[M][8];
#pragma unroll
    for (int jb = 0; jb < M; ++jb)
        load_a(jb, A[jb]);
    __syncthreads();   // qa's bytes are the code tiles from here on
    const uint32_t tcopy = (uint32_t)(uintptr_t)(lds_u8 *)ktable + (lane % NC) * EB;
    const uint32_t vcopy = (uint32_t)(uintptr_t)(lds_u8 *)vtable + (lane % kLdsCopies8) * 8;
    // after the hi/lo combine, lane l holds heads hu and hu + 2 of token l % 16
    const uint32_t hu = 4u * (part & 1u) + (lane >> 5);
    // scores in log2 units, so that every exponential is a bare 2^x
    const float pw_u = pw_s[hu] * kLog2e, pw_v = pw_s[hu + 2] * kLog2e;
    float *ft = ftile[wave];
    // this lane's 8-value field in a block of a token row of the code tile (column n:
    // values 8 n .. 8 n + 7): dwords dA, dA + 1 of the block's 12, shifted by fsh
    constexpr int FBITS = 8 * BITS;
    const uint32_t dA = (FBITS * n) >> 5, fsh = (FBITS * n) & 31u;
    // A rows: lane n of a lane group is row n = 8 hilo + 2 hh + e.  A token's four
    // k-slots take (yh of parity 0, yh of parity 1, yl of parity 0, yl of parity 1), so
    // its two A dwords are both (w, 0) for parity 0 and (0, w) for parity 1, w the hi or
    // lo half of the packed weight: one byte permute
    const uint32_t a_hh = (n >> 1) & 3u;
    const uint32_t sel_w = (n & 8u) ? 0x0C0C0302u : 0x0C0C0100u;
    const uint32_t a_sel = (n & 1u) ? ((sel_w << 16) | 0x0C0Cu) : sel_w;
    // after the hi/lo combine, lane l holds head hv of each set: rows 4 (l / 16) .. + 3
    // are heads 2 ((l / 16) & 1) and + 1, each at both parities
    const uint32_t hv = 2u * (part & 1u) + (lane >> 5);

    // online softmax state: running max and sum of heads hu, hu + 2 (the same in all 16
    // lanes of a row), the value-norm exponent E (wave-wide) and the P.V accumulators
    // (block jb, head set hs, product block c: rows 4 (lane / 16) .. + 3, column lane % 16)
    float m_u = -__builtin_inff(), m_v = -__builtin_inff(), l_u = 0.0f, l_v = 0.0f;
    int E = -1000;
    f4_t acc[M][NHS][4];
#pragma unroll
    for (int jb = 0; jb < M; ++jb)
#pragma unroll
        for (int hs = 0; hs < NHS; ++hs)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[jb][hs][c] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // batches of units k0 .. k0 + DEPTH - 1 (unit k0 holds a live row); the next
    // batch's norms are requested first, so that they are the oldest loads in flight
    // when that batch starts
    for (uint32_t k0 = 0; k0 < nunits; k0 += DEPTH) {
        prio_by_progress(k0, nunits);
        uint32_t nkn, nvn;
        fetch_norms(k0 + DEPTH, nkn, nvn);
        // scores of heads hu, hu + 2 for token n of each unit (as qk_kernel, summed over
        // the row's blocks), -inf past the range; the units' packed value codes into
        // their tiles (row n, block jb, bytes 4 BITS part ..)
        float su[DEPTH], sv[DEPTH], nvd[DEPTH][M];
        float bu = -__builtin_inff(), bv = -__builtin_inff(), bn = 0.0f;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            uint32_t *rt = raw_base + (d * kWavesPerGroup + wave) * kRawWords;
            f4_t sc = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            float nmax = 0.0f;
#pragma unroll
            for (int jb = 0; jb < M; ++jb) {
#pragma unroll
                for (int i = 0; i < LW; ++i)
                    rt[n * RW + 4 * BITS * jb + part * LW + i] = wv[d][jb][i];
                const int src = (16 * d + (int)n) * M + jb;   // the lane holding this norm
                const uint16_t nk16 = (uint16_t)__shfl((int)nkc, src, 64);
                const uint16_t nv16 = (uint16_t)__shfl((int)nvc, src, 64);
                const f4_t Du = qk_unit<BITS>(A[jb], wk[d][jb], tcopy);
                sc += Du * (float)__builtin_bit_cast(_Float16, nk16);
                nvd[d][jb] = (float)__builtin_bit_cast(_Float16, nv16);
                nmax = __builtin_fmaxf(nmax, nvd[d][jb]);
            }
            float s0 = sc[0], s1 = sc[1], s2 = sc[2], s3 = sc[3];
            swap32(s0, s1);
            swap32(s2, s3);
            const bool live = first + 16u * (k0 + d) + n < last;
            su[d] = live ? (s0 + s1) * pw_u : -__builtin_inff();
            sv[d] = live ? (s2 + s3) * pw_v : -__builtin_inff();
            bu = __builtin_fmaxf(bu, su[d]);
            bv = __builtin_fmaxf(bv, sv[d]);
            bn = __builtin_fmaxf(bn, live ? nmax : 0.0f);
            fetch(k0 + DEPTH + d, wk[d], wv[d]);
        }
        // online softmax over the batch's 64 / M rows (unit k0 holds a live row, so the
        // maxima are finite); the value-norm exponent follows the largest norm so far
        const float mu = __builtin_fmaxf(m_u, row16_max(bu));
        const float mv = __builtin_fmaxf(m_v, row16_max(bv));
        const float au = exp2_fast(m_u - mu), av = exp2_fast(m_v - mv);
        int eu = 0;
        (void)frexpf(row16_max(bn), &eu);
        const int En = max(E, __builtin_amdgcn_readfirstlane(eu));
        float ru = 0.0f, rv = 0.0f;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const float pu = exp2_fast(su[d] - mu), pv = exp2_fast(sv[d] - mv);
            ru += pu;
            rv += pv;
#pragma unroll
            for (int jb = 0; jb < M; ++jb) {
                uint32_t *pt = pt_base + ((d * M + jb) * kWavesPerGroup + wave) * (kQkHeads * 16);
                pt[hu * 16 + n] = split_pack(ldexpf(pu * nvd[d][jb], kAttnWExp - En));
                pt[(hu + 2) * 16 + n] = split_pack(ldexpf(pv * nvd[d][jb], kAttnWExp - En));
            }
        }
        l_u = l_u * au + row16_sum(ru);
        l_v = l_v * av + row16_sum(rv);
        m_u = mu;
        m_v = mv;
        const bool resc = __any(au != 1.0f || av != 1.0f) || En != E;
        if (resc) {   // scale acc rows by their head's exp(m_old - m_new) 2^(E_old - E_new)
            const float sE = ldexpf(1.0f, E - En);
            if (n == 0) {
                ft[hu] = au * sE;
                ft[hu + 2] = av * sE;
            }
            wave_lds_sync();
#pragma unroll
            for (int hs = 0; hs < NHS; ++hs) {
                const float2 f2 = *(const float2 *)(ft + 4 * hs + 2 * (part & 1u));
                const f4_t f4 = f4_t{f2.x, f2.x, f2.y, f2.y};
#pragma unroll
                for (int jb = 0; jb < M; ++jb)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[jb][hs][c] = acc[jb][hs][c] * f4;
            }
        }
        E = En;
        wave_lds_sync();   // weights and code tiles complete
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint32_t *rt = raw_base + (d * kWavesPerGroup + wave) * kRawWords;
#pragma unroll
            for (int jb = 0; jb < M; ++jb) {
                const uint32_t *pt = pt_base + ((d * M + jb) * kWavesPerGroup + wave) * (kQkHeads * 16);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    // B: positions 8 n + 2 c, + 1 of tokens 8 kb + 2 part, + 1 (one lookup each)
                    uint64_t ent[2][4];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint32_t *row = rt + (8 * kb + 2 * part + j) * RW + 4 * BITS * jb + dA;
                        const uint32_t f = __builtin_amdgcn_alignbit(row[1], row[0], fsh);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint32_t e = __builtin_amdgcn_ubfe(f, 2 * BITS * c, 2 * BITS);
                            ent[j][c] = lds_load<uint64_t>(lshl_add<8>(e, vcopy));
                        }
                    }
#pragma unroll
                    for (int hs = 0; hs < NHS; ++hs) {
                        // A: the weights of head 4 hs + a_hh, tokens 8 kb + 2 part, + 1
                        const uint2 x = *(const uint2 *)(pt + (4 * hs + a_hh) * 16 + 8 * kb + 2 * part);
                        const uint32_t a0 = __builtin_amdgcn_perm(x.x, x.x, a_sel);
                        const uint32_t a1 = __builtin_amdgcn_perm(x.y, x.y, a_sel);
                        const u4_t av = u4_t{a0, a0, a1, a1};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const u4_t bv = u4_t{(uint32_t)ent[0][c], (uint32_t)(ent[0][c] >> 32),
                                                 (uint32_t)ent[1][c], (uint32_t)(ent[1][c] >> 32)};
                            acc[jb][hs][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(h8_t, av), __builtin_bit_cast(h8_t, bv),
                                acc[jb][hs][c], 0, 0, 0);
                        }
                    }
                }
            }
        }
        nkc = nkn;
        nvc = nvn;
    }

    // this wave's state into LDS (over the tables), then merged: rows r (hi) and r + 8
    // (lo) of acc sit in lanes l and l + 32; after the combine lane l holds positions
    // 8 n .. 8 n + 7 of block jb of head 4 s + hv
    __syncthreads();   // every wave is done with the tables
    float *mg = (float *)smem;   // [wave][head][acc[128 M], m, l, -, -]
#pragma unroll
    for (int jb = 0; jb < M; ++jb)
#pragma unroll
        for (int hs = 0; hs < NHS; ++hs) {
            float o[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float a0 = acc[jb][hs][c][0], a1 = acc[jb][hs][c][1];
                float a2 = acc[jb][hs][c][2], a3 = acc[jb][hs][c][3];
                swap32(a0, a2);
                swap32(a1, a3);
                o[2 * c] = ldexpf(a0 + a2, E - kAttnWExp);
                o[2 * c + 1] = ldexpf(a1 + a3, E - kAttnWExp);
            }
            float *r = mg + (wave * kQkHeads + 4 * hs + hv) * REC + kBlock * jb + 8 * n;
            *(float4 *)r = float4{o[0], o[1], o[2], o[3]};
            *(float4 *)(r + 4) = float4{o[4], o[5], o[6], o[7]};
        }
    if (n == 0) {
        float *ru = mg + (wave * kQkHeads + hu) * REC + kBlock * M;
        float *rv = mg + (wave * kQkHeads + hu + 2) * REC + kBlock * M;
        ru[0] = m_u;
        ru[1] = l_u;
        rv[0] = m_v;
        rv[1] = l_v;
    }
    __syncthreads();
    {
        // thread -> head threadIdx / 32, values 4 (threadIdx % 32) .. + 3 of every block
        const uint32_t h = threadIdx.x >> 5, v0 = 4u * (threadIdx.x & 31u);
        float Mx = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w)
            Mx = __builtin_fmaxf(Mx, mg[(w * kQkHeads + h) * REC + kBlock * M]);
        float L = 0.0f, a[M][4];
#pragma unroll
        for (int jb = 0; jb < M; ++jb)
            a[jb][0] = a[jb][1] = a[jb][2] = a[jb][3] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) {
            const float *r = mg + (w * kQkHeads + h) * REC;
            const float f = r[kBlock * M] == -__builtin_inff() ? 0.0f : exp2_fast(r[kBlock * M] - Mx);
            L += f * r[kBlock * M + 1];
#pragma unroll
            for (int jb = 0; jb < M; ++jb) {
                const float4 x = *(const float4 *)(r + kBlock * jb + v0);
                a[jb][0] += f * x.x;
                a[jb][1] += f * x.y;
                a[jb][2] += f * x.z;
                a[jb][3] += f * x.w;
            }
        }
        if (h < nh) {
            float *rec = work + (((size_t)b * Hq + h0 + h) * nparts + blockIdx.y) * REC;
#pragma unroll
            for (int jb = 0; jb < M; ++jb)
                *(float4 *)(rec + 4 + kBlock * jb + v0) = float4{a[jb][0], a[jb][1], a[jb][2], a[jb][3]};
            if (v0 == 0) {
                rec[0] = Mx;
                rec[1] = L;
            }
        }
    }
}

// One workgroup per (sequence, query head): merge the chunks' partials (wave w takes
// chunks w, w + 4, ...; lane l values l and 64 + l of every block), add the four waves,
// transform each block once and divide by 128 l.
template <int M>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float *__restrict__ work,
                                                           float *__restrict__ out,
                                                           uint32_t nparts, Signs sg)
{
    constexpr int REC = attn_rec(M);
    __shared__ float red[kWavesPerGroup][kBlock * M + 1];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t bh = blockIdx.x;
    const float *rec = work + (size_t)bh * nparts * REC;
    // the largest running max over all chunks (every wave computes it)
    float Mx = -__builtin_inff();
    for (uint32_t p = lane; p < nparts; p += 64)
        Mx = __builtin_fmaxf(Mx, rec[(size_t)p * REC]);
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1)
        Mx = __builtin_fmaxf(Mx, __shfl_xor(Mx, h, 64));
    float L = 0.0f, a[M], c[M];
#pragma unroll
    for (int jb = 0; jb < M; ++jb)
        a[jb] = c[jb] = 0.0f;
#pragma unroll 4
    for (uint32_t p = wave; p < nparts; p += kWavesPerGroup) {
        const float *r = rec + (size_t)p * REC;
        const float w = exp2_fast(r[0] - Mx);   // every chunk holds a row: r[0] is finite
        L += w * r[1];
#pragma unroll
        for (int jb = 0; jb < M; ++jb) {
            a[jb] += w * r[4 + kBlock * jb + lane];
            c[jb] += w * r[68 + kBlock * jb + lane];
        }
    }
#pragma unroll
    for (int jb = 0; jb < M; ++jb) {
        red[wave][kBlock * jb + lane] = a[jb];
        red[wave][kBlock * jb + 64 + lane] = c[jb];
    }
    if (lane == 0)
        red[wave][kBlock * M] = L;
    __syncthreads();
    if (wave != 0)
        return;
    L = red[0][kBlock * M] + red[1][kBlock * M] + red[2][kBlock * M] + red[3][kBlock * M];
    const float inv = 1.0f / (128.0f * L);
#pragma unroll
    for (int jb = 0; jb < M; ++jb) {
        const uint32_t o = kBlock * jb;
        float x = red[0][o + lane] + red[1][o + lane] + red[2][o + lane] + red[3][o + lane];
        float y = red[0][o + 64 + lane] + red[1][o + 64 + lane] + red[2][o + 64 + lane] +
                  red[3][o + 64 + lane];
        // H: span 64 in-lane, spans 32..1 across lanes
        const float s0 = x + y;
        y = x - y;
        x = s0;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {
            const float px = __shfl_xor(x, h, 64), py = __shfl_xor(y, h, 64);
            const bool up = (lane & (uint32_t)h) != 0u;
            x = up ? px - x : x + px;
            y = up ? py - y : y + py;
        }
        // D H acc / (128 l): the randomised rotation's signs flip the output positions
        const uint32_t ux = __builtin_bit_cast(uint32_t, x * inv) ^ sign_mask_f32(sg, lane);
        const uint32_t uy = __builtin_bit_cast(uint32_t, y * inv) ^ sign_mask_f32(sg, 64u + lane);
        out[(size_t)bh * kBlock * M + o + lane] = __builtin_bit_cast(float, ux);
        out[(size_t)bh * kBlock * M + o + 64 + lane] = __builtin_bit_cast(float, uy);
    }
}

// ---------------------------------------------------------------- interleaved records
//
// A block as one record of 2 + 16 BITS bytes: its fp16 norm (little-endian), then its
// code bytes, records in block order (each block packs 128 values and one FP16 norm,
// 50 / 34 bytes: the article's size section).  Both directions are byte moves bound
// by HBM: a wave takes a tile of 64 blocks, reads it with 16-byte loads into LDS, and
// writes the other layout with 16-byte stores, gathering halfwords from LDS (records
// are 2-byte granular).  A tile of 64 records starts 16-byte aligned (64 x 50 and 64 x
// 34 are multiples of 16); the last tile's ragged end goes out halfword by halfword.

constexpr int kRecTile = 64;   // blocks per wave tile

template <int BITS>
__global__ __launch_bounds__(256) void pack_records_kernel(const uint8_t *__restrict__ codes,
                                                           const uint16_t *__restrict__ norms,
                                                           uint32_t nblocks,
                                                           uint8_t *__restrict__ rec)
{
    constexpr int CB = 16 * BITS, RH = CB / 2 + 1;   // code bytes, halfwords per record
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[kWavesPerGroup][kRecTile * (CB + 2)];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t b0 = (blockIdx.x * kWavesPerGroup + wave) * kRecTile;
    if (b0 >= nblocks)
        return;
    const uint32_t nb = min(nblocks - b0, (uint32_t)kRecTile);
    uint8_t *lc = lds_all[wave];                              // codes [64][CB]
    uint16_t *ln = (uint16_t *)(lc + kRecTile * CB);          // norms [64]
    const u4_t *src = (const u4_t *)(codes + (size_t)b0 * CB);
    const uint32_t nch = nb * (CB / 16);
    for (uint32_t c = lane; c < nch; c += 64u)
        *(u4_t *)(lc + c * 16u) = ld_stream(src + c);
    if (lane < nb)
        ln[lane] = ld_stream(norms + b0 + lane);
    wave_lds_sync();

    const uint16_t *lc16 = (const uint16_t *)lc;
    const uint32_t nh = nb * RH;                              // halfwords of the tile's records
    uint8_t *dst = rec + (size_t)b0 * (CB + 2);
    for (uint32_t h = 8u * lane; h < nh; h += 512u) {
        uint32_t r = h / RH, k = h - r * RH;
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = h + i < nh ? (k == 0 ? ln[r] : lc16[r * (CB / 2) + k - 1]) : 0u;
            if (++k == (uint32_t)RH) {
                k = 0;
                ++r;
            }
        }
        if (h + 8u <= nh) {
            *(u4_t *)(dst + 2u * h) = u4_t{v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16,
                                           v[6] | v[7] << 16};
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (h + i < nh)
                    ((uint16_t *)dst)[h + i] = (uint16_t)v[i];
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void unpack_records_kernel(const uint8_t *__restrict__ rec,
                                                             uint32_t nblocks,
                                                             uint8_t *__restrict__ codes,
                                                             uint16_t *__restrict__ norms)
{
    constexpr int CB = 16 * BITS, RH = CB / 2 + 1;
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[kWavesPerGroup][kRecTile * (CB + 2)];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t b0 = (blockIdx.x * kWavesPerGroup + wave) * kRecTile;
    if (b0 >= nblocks)
        return;
    const uint32_t nb = min(nblocks - b0, (uint32_t)kRecTile);
    uint8_t *lr = lds_all[wave];
    const uint8_t *srcb = rec + (size_t)b0 * (CB + 2);
    const uint32_t nh = nb * RH, nfull = nh / 8u;             // whole 16-byte chunks, then halfwords
    for (uint32_t c = lane; c < nfull; c += 64u)
        *(u4_t *)(lr + c * 16u) = ld_stream((const u4_t *)srcb + c);
    if (8u * nfull + lane < nh)
        ((uint16_t *)lr)[8u * nfull + lane] = ld_stream((const uint16_t *)srcb + 8u * nfull + lane);
    wave_lds_sync();

    const uint16_t *lr16 = (const uint16_t *)lr;
    constexpr uint32_t CPB = CB / 16;                         // 16-byte code chunks per block
    uint8_t *dstc = codes + (size_t)b0 * CB;
    for (uint32_t c = lane; c < nb * CPB; c += 64u) {
        const uint32_t r = c / CPB, j = c - r * CPB;
        const uint16_t *p = lr16 + r * RH + 1u + 8u * j;
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = p[i];
        *(u4_t *)(dstc + 16u * c) = u4_t{v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16,
                                         v[6] | v[7] << 16};
    }
    if (lane < nb)
        norms[b0 + lane] = lr16[lane * RH];
}

// Compute units of the current device (cached per device; threads that race on the
// first call store the same value).
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Cap on workgroups per compute unit of a codec grid, 0 for none, overridable for
// tuning sweeps with TQ_ENCODE_GROUPS_PER_CU, TQ_ENCODE_ROT_GROUPS_PER_CU and
// TQ_DECODE_GROUPS_PER_CU.
//   encode: no cap, one 32-block tile per wave.  The hardware then starts a new
//     workgroup whenever one retires (126 VGPRs and 6 KB of LDS allow four per CU),
//     so the waves' load, compute and store phases drift apart.  A persistent grid
//     of two groups per CU, each wave prefetching its next tile, runs the same
//     eight-layer encode at 5.28 TB/s against 5.6 TB/s for this one (8 to 24 layers
//     gain 3-7 %, one layer is unchanged).  The randomised-rotation variant needs
//     its sign masks too: with the tile loop (a capped grid) that takes it to 142
//     VGPRs, three waves per SIMD, so a grid of one tile per wave launches its build
//     without the loop (LOOP = false: no load registers kept for a next tile, 105
//     VGPRs, four waves per SIMD), 11-16 % faster than the capped loop.  The plain
//     encoder's loop-free build (72 VGPRs) measured no faster than the loop at
//     126, so it always runs the loop.
//   decode: no cap either, one 32-block tile per wave (80-106 VGPRs and 20 / 33 KB of
//     LDS allow four to six groups per CU); caps of 5, 10 or 20 groups per CU
//     measured slower on 8- to 48-layer caches.
int groups_per_cu(const char *env, int dflt)
{
    const char *e = getenv(env);
    int v = e ? atoi(e) : -1;
    return v >= 0 && v <= 4096 ? v : dflt;
}

// Grid of a strided codec kernel: enough groups to give every wave one tile, at
// most `per_cu` groups per CU (per_cu 0: no cap) and at most 2^22 groups (2^30
// work-items, inside the launch limit of 2^32; larger inputs take several tiles
// per wave).
inline int grid_for(int64_t nblocks, int tile_blocks, int per_cu)
{
    const int64_t per_group = (int64_t)kWavesPerGroup * tile_blocks;
    int64_t n = (nblocks + per_group - 1) / per_group;
    if (per_cu > 0 && n > (int64_t)cu_count() * per_cu)
        n = (int64_t)cu_count() * per_cu;
    return (int)(n < ((int64_t)1 << 22) ? n : ((int64_t)1 << 22));
}

}  // namespace

static bool has_signs(const Signs &sg) { return (sg.w[0] | sg.w[1] | sg.w[2] | sg.w[3]) != 0u; }

// Timing hook: start / stop events for the next kernel this thread launches.
static thread_local hipEvent_t next_start = nullptr, next_stop = nullptr;

void set_next_launch_events(void *start, void *stop)
{
    next_start = (hipEvent_t)start;
    next_stop = (hipEvent_t)stop;
}

// Every kernel launch goes through here: a plain launch, or, when the timing hook is
// set, one whose dispatch packet itself records the start and stop timestamps
// (hipExtLaunchKernelGGL), after which the hook is cleared.
template <typename F, typename... Args>
static void launch_kernel(F kern, dim3 grid, dim3 block, uint32_t smem, hipStream_t s,
                          Args... args)
{
    if (next_start || next_stop) {
        hipEvent_t a = next_start, b = next_stop;
        next_start = next_stop = nullptr;
        hipExtLaunchKernelGGL(kern, grid, block, smem, s, a, b, 0u, args...);
    } else {
        hipLaunchKernelGGL(kern, grid, block, smem, s, args...);
    }
}

int launch_encode(int bits, const Signs &sg, const void *x, int64_t nblocks, int64_t row_blocks,
                  int64_t cache_row_blocks, int64_t t0_blocks, void *codes, void *norms,
                  void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    static const int per_cu = groups_per_cu("TQ_ENCODE_GROUPS_PER_CU", 0);
    static const int per_cu_rot = groups_per_cu("TQ_ENCODE_ROT_GROUPS_PER_CU", 0);
    const bool rot = has_signs(sg);
    dim3 grid(grid_for(nblocks, kEncTileBlocks, rot ? per_cu_rot : per_cu)), block(256);
    auto launch = [&](auto kern) {
        launch_kernel(kern, grid, block, 0, s, (const uint8_t *)x, (uint32_t)nblocks,
                      (uint32_t)row_blocks, cache_row_blocks, t0_blocks, (uint8_t *)codes,
                      (uint16_t *)norms, *cb, sg);
    };
    const bool loop = (int64_t)grid.x * kWavesPerGroup * kEncTileBlocks < nblocks;
    if (bits == 3) {
        if (rot)
            loop ? launch(encode_kernel<3, true, true>) : launch(encode_kernel<3, true, false>);
        else
            launch(encode_kernel<3, false, true>);
    } else {
        if (rot)
            loop ? launch(encode_kernel<2, true, true>) : launch(encode_kernel<2, true, false>);
        else
            launch(encode_kernel<2, false, true>);
    }
    return (int)hipGetLastError();
}

int launch_decode(int bits, const Signs &sg, const void *codes, const void *norms,
                  int64_t nblocks, int64_t row_blocks, int64_t cache_row_blocks,
                  int64_t t0_blocks, void *x, void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    static const int per_cu = groups_per_cu("TQ_DECODE_GROUPS_PER_CU", 0);
    dim3 grid(grid_for(nblocks, kEncTileBlocks, per_cu)), block(256);
    auto launch = [&](auto kern) {
        launch_kernel(kern, grid, block, 0, s, (const uint8_t *)codes, (const uint16_t *)norms,
                      (uint32_t)nblocks, (uint32_t)row_blocks, cache_row_blocks, t0_blocks,
                      (uint8_t *)x, *cb, sg);
    };
    const bool rot = has_signs(sg);
    if (bits == 3)
        rot ? launch(decode_kernel<3, true>) : launch(decode_kernel<3, false>);
    else
        rot ? launch(decode_kernel<2, true>) : launch(decode_kernel<2, false>);
    return (int)hipGetLastError();
}

int launch_qk(int bits, const Signs &sg, const void *k_codes, const void *k_norms, int64_t B,
              int64_t Hkv, int64_t Tc, int64_t m, int64_t T, const void *q, int64_t Hq,
              float scale, float *scores, void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    const int64_t G = Hq / Hkv;
    const int64_t passes = (G + kQkHeads - 1) / kQkHeads;
    // Rows per workgroup: about one round of workgroups (kQkGroupsPerCu per CU, the
    // kernel's occupancy) so each pays its table and query prologue once, whole
    // batches of kQkDepth units per wave, at most 65535 row chunks.
    const int64_t step = (int64_t)kWavesPerGroup * 16 * (m >= kQkDepth ? 1 : kQkDepth / m);
    const int64_t pairs = B * Hkv * passes;
    const int64_t round = (int64_t)cu_count() * qk_groups_per_cu(bits, m);
    int64_t tpg = (T * pairs + round - 1) / round;
    tpg = tpg < (T + 65534) / 65535 ? (T + 65534) / 65535 : tpg;
    tpg = ((tpg + step - 1) / step) * step;
    if (tpg < step)
        tpg = step;
    if (tpg > 8192)
        tpg = ((8192 + step - 1) / step) * step;
    if ((T + tpg - 1) / tpg > 65535)
        tpg = (((T + 65534) / 65535 + step - 1) / step) * step;
    dim3 grid((uint32_t)pairs, (uint32_t)((T + tpg - 1) / tpg));
    dim3 block(256);
    const size_t smem = qk_smem_bytes(bits, m);
    auto launch = [&](auto kern) -> int {
        if (smem > 65536) {
            hipError_t e = hipFuncSetAttribute((const void *)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            if (e != hipSuccess)
                return (int)e;
        }
        launch_kernel(kern, grid, block, smem, s, (const uint8_t *)k_codes,
                      (const uint16_t *)k_norms, (const uint16_t *)q, scores, (uint32_t)Hkv,
                      Tc, (uint32_t)T, (uint32_t)m, (uint32_t)G, (uint32_t)Hq,
                      (uint32_t)passes, (uint32_t)tpg, scale, *cb, sg);
        return (int)hipGetLastError();
    };
    if (bits == 3)
        return m == 1 ? launch(qk_kernel<3, 1>) : m == 2 ? launch(qk_kernel<3, 2>) : launch(qk_kernel<3, 0>);
    return m == 1 ? launch(qk_kernel<2, 1>) : m == 2 ? launch(qk_kernel<2, 2>) : launch(qk_kernel<2, 0>);
}


int launch_pack_records(int bits, const void *codes, const void *norms, int64_t nblocks,
                        void *records, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const int64_t tiles = (nblocks + kRecTile - 1) / kRecTile;
    dim3 grid((uint32_t)((tiles + kWavesPerGroup - 1) / kWavesPerGroup)), block(256);
    if (bits == 3)
        launch_kernel(pack_records_kernel<3>, grid, block, 0, s, (const uint8_t *)codes,
                      (const uint16_t *)norms, (uint32_t)nblocks, (uint8_t *)records);
    else
        launch_kernel(pack_records_kernel<2>, grid, block, 0, s, (const uint8_t *)codes,
                      (const uint16_t *)norms, (uint32_t)nblocks, (uint8_t *)records);
    return (int)hipGetLastError();
}

int launch_unpack_records(int bits, const void *records, int64_t nblocks, void *codes,
                          void *norms, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const int64_t tiles = (nblocks + kRecTile - 1) / kRecTile;
    dim3 grid((uint32_t)((tiles + kWavesPerGroup - 1) / kWavesPerGroup)), block(256);
    if (bits == 3)
        launch_kernel(unpack_records_kernel<3>, grid, block, 0, s, (const uint8_t *)records,
                      (uint32_t)nblocks, (uint8_t *)codes, (uint16_t *)norms);
    else
        launch_kernel(unpack_records_kernel<2>, grid, block, 0, s, (const uint8_t *)records,
                      (uint32_t)nblocks, (uint8_t *)codes, (uint16_t *)norms);
    return (int)hipGetLastError();
}

// Decode attention chunking, from the sizes alone (tq_attn_workspace_bytes needs no
// device): about attn_groups_per_cu workgroups per CU of a 256-CU MI355X (two head sets
// when G > 4, as the launch picks its kernel), whole batches of attn_depth(m) units per
// wave, at most 65535 chunks.
int64_t attn_chunk_rows(int bits, int64_t B, int64_t Hkv, int64_t T, int64_t Hq, int64_t m)
{
    const int64_t G = Hq / Hkv, passes = (G + kQkHeads - 1) / kQkHeads;
    const int64_t step = (int64_t)kWavesPerGroup * 16 * attn_depth((int)m);
    const int64_t round = 256 * attn_groups_per_cu(bits, G > kQkHeads / 2 ? 2 : 1, (int)m);
    int64_t rows = (T * B * Hkv * passes + round - 1) / round;
    rows = rows < (T + 65534) / 65535 ? (T + 65534) / 65535 : rows;
    rows = ((rows + step - 1) / step) * step;
    return rows < step ? step : rows;
}

// Workspace of tq_attn_decode_noalloc: a file-scope device array, one copy per device
// (created when the code object is loaded there, held until the process ends).  Host
// code never uses its name as an address: attn_scratch() looks the device address up.
static __device__ __align__(256) uint8_t scratch[TQ_ATTN_SCRATCH_BYTES];

void *attn_scratch()
{
    static std::atomic<void *> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {   // first call on this device, which is current: its own copy's address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        cache[dev].store(p, std::memory_order_release);
    }
    return p;
}

int64_t attn_workspace_bytes(int bits, int64_t B, int64_t Hkv, int64_t T, int64_t Hq, int64_t m)
{
    const int64_t rows = attn_chunk_rows(bits, B, Hkv, T, Hq, m);
    const int64_t chunks = (T + rows - 1) / rows;
    return B * Hq * chunks * attn_rec((int)m) * (int64_t)sizeof(float);
}

int launch_attn(int bits, const Signs &sg, const void *k_codes, const void *k_norms,
                const void *v_codes, const void *v_norms, int64_t B, int64_t Hkv, int64_t Tc,
                int64_t m, int64_t T, const void *q, int64_t Hq, float scale, float *out,
                void *work, void *stream)
{
    const Codebook *cb = codebook(bits);
    hipStream_t s = (hipStream_t)stream;
    const int64_t G = Hq / Hkv, passes = (G + kQkHeads - 1) / kQkHeads;
    const int64_t rows = attn_chunk_rows(bits, B, Hkv, T, Hq, m);
    const int64_t chunks = (T + rows - 1) / rows;
    const uint32_t nparts = (uint32_t)chunks;
    dim3 grid((uint32_t)(B * Hkv * passes), (uint32_t)chunks), block(256);
    auto partial = [&](auto kern) {
        launch_kernel(kern, grid, block, 0, s, (const uint8_t *)k_codes, (const uint16_t *)k_norms,
                      (const uint8_t *)v_codes, (const uint16_t *)v_norms, (const uint16_t *)q,
                      (float *)work, (uint32_t)Hkv, Tc, (uint32_t)T, (uint32_t)G, (uint32_t)Hq,
                      (uint32_t)passes, (uint32_t)rows, nparts, scale, *cb, sg);
    };
    if (m == 1) {
        if (bits == 3)
            G > 4 ? partial(attn_partial_kernel<3, 2, 1>) : partial(attn_partial_kernel<3, 1, 1>);
        else
            G > 4 ? partial(attn_partial_kernel<2, 2, 1>) : partial(attn_partial_kernel<2, 1, 1>);
    } else {
        if (bits == 3)
            G > 4 ? partial(attn_partial_kernel<3, 2, 2>) : partial(attn_partial_kernel<3, 1, 2>);
        else
            G > 4 ? partial(attn_partial_kernel<2, 2, 2>) : partial(attn_partial_kernel<2, 1, 2>);
    }
    int e = (int)hipGetLastError();
    if (e)
        return e;
    if (m == 1)
        launch_kernel(attn_combine_kernel<1>, dim3((uint32_t)(B * Hq)), dim3(256), 0, s,
                      (const float *)work, out, nparts, sg);
    else
        launch_kernel(attn_combine_kernel<2>, dim3((uint32_t)(B * Hq)), dim3(256), 0, s,
                      (const float *)work, out, nparts, sg);
    return (int)hipGetLastError();
}

}  // namespace tq
