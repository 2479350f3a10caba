// internal.h -- declarations shared by the library's own translation units
// (host C-ABI layer, codebook set-up and the gfx950 kernels).  Not installed,
// not part of the C ABI.
#pragma once

#include <stdint.h>

namespace tq {

constexpr int kBlock = 128;          // values per block
constexpr int kWave = 64;            // gfx950 wavefront size
constexpr int kWavesPerGroup = 4;    // 256-thread workgroups

// float32 constants of one cache type, produced on the host from the N(0,1)
// Lloyd-Max conditions and handed to the kernels by value.
struct Codebook {
    int bits;              // 2 or 3
    float levels[8];       // ascending; code k -> levels[k]
    float thresholds[7];   // midpoints of adjacent levels
    // Encoder decision function.  With t = u / n the normalised rotated value,
    //   F(t) = 2^bits/2 + g(clamp(t, -clamp_t, clamp_t)),  code = floor(F),
    //   g(t) = t * (g1 + g2 |t| + g3 t^2)
    // odd, and increasing on [-clamp_t, clamp_t], with g(tau_k) = k at every
    // positive threshold tau_k (k = 1 .. 2^bits/2 - 1), so floor(F) counts the
    // thresholds at or below t.  For two bits g is linear (g1 = 1 / tau_1).
    float g1, g2, g3;
    float clamp_t;         // |g(clamp_t)| < 2^bits/2, so F stays in [0, 2^bits)
};

// The codebook of a type (2 or 3); nullptr for any other value.  Computed
// once per process, thread-safe.
const Codebook *codebook(int bits);

// Signs of the randomised rotation H D: bit p % 32 of w[p / 32] set <=> D_pp = -1
// (all zero: the plain H).  Handed to the kernels by value.
struct Signs {
    uint32_t w[4];
};

// Kernel launchers (asynchronous on `stream`).  Each returns 0 on a clean
// launch and a nonzero HIP error code otherwise.  Shapes are pre-validated.
// The next kernel launched by this thread records its own start / stop on these
// hipEvent_t (null: no event); the hook then clears itself.
void set_next_launch_events(void *start, void *stop);

int launch_encode(int bits, const Signs &sg, const void *x, int64_t nblocks, int64_t row_blocks,
                  int64_t cache_row_blocks, int64_t t0_blocks, void *codes, void *norms,
                  void *stream);
int launch_decode(int bits, const Signs &sg, const void *codes, const void *norms,
                  int64_t nblocks, int64_t row_blocks, int64_t cache_row_blocks,
                  int64_t t0_blocks, void *x, void *stream);
int launch_qk(int bits, const Signs &sg, const void *k_codes, const void *k_norms, int64_t B,
              int64_t Hkv, int64_t Tc, int64_t m, int64_t T, const void *q, int64_t Hq,
              float scale, float *scores, void *stream);

// Decode attention (D = 128 m, m = 1 or 2): rows per chunk and workspace bytes follow
// from the sizes alone; the launch runs the partial and the combine kernel.
int64_t attn_chunk_rows(int bits, int64_t B, int64_t Hkv, int64_t T, int64_t Hq, int64_t m);
int64_t attn_workspace_bytes(int bits, int64_t B, int64_t Hkv, int64_t T, int64_t Hq, int64_t m);
int launch_attn(int bits, const Signs &sg, const void *k_codes, const void *k_norms,
                const void *v_codes, const void *v_norms, int64_t B, int64_t Hkv, int64_t Tc,
                int64_t m, int64_t T, const void *q, int64_t Hq, float scale, float *out,
                void *work, void *stream);
// Device address of the current device's static attention scratch array (looked up
// once per device), or nullptr when HIP cannot report it.
void *attn_scratch();

// Interleaved records (2 + 16 bits bytes per block) from / to the two planes,
// nblocks < 2^31.
int launch_pack_records(int bits, const void *codes, const void *norms, int64_t nblocks,
                        void *records, void *stream);
int launch_unpack_records(int bits, const void *records, int64_t nblocks, void *codes,
                          void *norms, void *stream);

}  // namespace tq
