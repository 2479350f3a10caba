"""Bounds of the fused read kernels' memory accesses, replayed on the CPU.

The q.K kernel, the decode attention's partial kernel and its combine kernel compute
every global address from the launch shape, the workgroup and lane indices and a
few clamps.  A mistake there faults the GPU (a q.K store past the last query head
of a pass once did: the score lines of lanes whose head lay beyond the pass were
written to the next sequence's rows, and beyond the buffer for the last one; the
kernel now clamps those lanes to the pass's last head).  This test restates that
arithmetic -- the host's grid and chunking, each wave's row range, the clamped
code / norm / query loads, the score stores of both loops, the attention's LDS
tiles and workspace records, the combine's reads and writes -- and checks, for
every lane of every workgroup, that each access stays inside its buffer, for every
shape the GPU tests, the smoke check, the quality harness and the benchmark launch.
The constants it assumes are read back from kernels.hip, so a change there that the
replay does not follow fails here.  It also replays which tiles the encoder's waves
take (turbo2 reorders them), and checks that every tile is encoded exactly once.
"""
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = os.path.join(ROOT, "kv_cache_quantization_block_amd", "csrc", "kernels.hip")
INTERNAL = os.path.join(ROOT, "kv_cache_quantization_block_amd", "csrc", "internal.h")

# constants of the kernels this replay assumes
WAVES = 4                 # kWavesPerGroup
QK_DEPTH = 4              # kQkDepth
QK_HEADS = 8              # kQkHeads
QK_GROUPS_PER_CU = 4      # kQkGroupsPerCu
# attn_groups_per_cu(bits, NHS, M), NHS = sets of four query heads (2 when G > 4)
ATTN_GROUPS = {(3, 1, 1): 4, (3, 2, 1): 3, (2, 1, 1): 3, (2, 2, 1): 3,
               (3, 1, 2): 2, (3, 2, 2): 2, (2, 1, 2): 2, (2, 2, 2): 2}


def test_constants_match_the_kernels():
    src = open(KERNELS).read() + open(INTERNAL).read()

    def const(name):
        m = re.search(r"constexpr int %s = (\d+);" % name, src)
        assert m, name
        return int(m.group(1))

    assert const("kWavesPerGroup") == WAVES
    assert const("kQkDepth") == QK_DEPTH
    assert const("kQkHeads") == QK_HEADS
    assert const("kQkGroupsPerCu") == QK_GROUPS_PER_CU
    assert "return M == 2 ? 2 : bits == 3 && NHS == 1 ? 4 : 3;" in src
    assert "const int64_t round = 256 * attn_groups_per_cu(bits, G > kQkHeads / 2 ? 2 : 1, (int)m);" in src
    assert "constexpr int RW = 4 * BITS * M;" in src
    assert "constexpr int attn_depth(int M) { return 4 / M; }" in src
    assert "constexpr int attn_rec(int M) { return 4 + kBlock * M; }" in src
    assert "if (tpg > 8192)" in src and "65535" in src
    assert "return m == 2 ? 3 : bits == 3 && m == 1 ? 5 : kQkGroupsPerCu;" in src
    # q.K's prefetch clamp, as replayed below
    assert "const uint32_t lastc = first < last ? last - 1u : t_end - 1u;" in src
    assert "const uint32_t tb = min(first + gi * 16u, lastc);" in src
    assert "const size_t emax = (row0 + lastc) * MD + (MD - 1u);" in src
    assert "const int64_t round = (int64_t)cu_count() * qk_groups_per_cu(bits, m);" in src
    assert "na = ld_stream(k_norms + min(e0 + lane, emax));" in src


def cdiv(a, b):
    return -(-a // b)


def rup(a, b):
    return cdiv(a, b) * b


class Buf:
    """Bounds of one buffer, in elements: records the accesses' range."""

    def __init__(self, name, size):
        self.name, self.size, self.n = name, int(size), 0

    def check(self, idx, width=1, mask=None, align=1):
        idx = np.asarray(idx, dtype=np.int64)
        if mask is not None:
            idx = idx[np.broadcast_to(mask, idx.shape)]
        if idx.size == 0:
            return
        lo, hi = int(idx.min()), int(idx.max()) + width - 1
        assert lo >= 0 and hi < self.size, f"{self.name}: [{lo}, {hi}] outside [0, {self.size})"
        if align > 1:
            assert np.all(idx % align == 0), f"{self.name}: misaligned access"
        self.n += idx.size


LANE = np.arange(64, dtype=np.int64)
N16, PART = LANE & 15, LANE >> 4


# ---------------------------------------------------------------- q.K

def qk_groups_per_cu(bits, m):
    return 3 if m == 2 else 5 if bits == 3 and m == 1 else QK_GROUPS_PER_CU


def qk_grid(bits, B, Hkv, T, m, Hq, cu):
    G = Hq // Hkv
    passes = cdiv(G, QK_HEADS)
    step = WAVES * 16 * (1 if m >= QK_DEPTH else QK_DEPTH // m)
    pairs = B * Hkv * passes
    rnd = cu * qk_groups_per_cu(bits, m)
    tpg = cdiv(T * pairs, rnd)
    tpg = max(tpg, cdiv(T, 65535))
    tpg = max(rup(tpg, step), step)
    if tpg > 8192:
        tpg = rup(8192, step)
    if cdiv(T, tpg) > 65535:
        tpg = rup(cdiv(T, 65535), step)
    return G, passes, pairs, cdiv(T, tpg), tpg


def wave_contexts(nx, ny, passes, Hkv, G, T, Tc, rows):
    """Arrays over (workgroup x, workgroup y, wave) of the per-wave quantities both
    kernels compute the same way."""
    x, y, w = np.meshgrid(np.arange(nx), np.arange(ny), np.arange(WAVES), indexing="ij")
    x, y, w = x.reshape(-1, 1), y.reshape(-1, 1), w.reshape(-1, 1)
    c = dict(x=x, y=y, wave=w)
    c["pass"] = x % passes
    c["bg"] = x // passes
    c["b"], c["g"] = c["bg"] // Hkv, c["bg"] % Hkv
    c["h0"] = c["g"] * G + c["pass"] * QK_HEADS
    c["nh"] = np.minimum(G - c["pass"] * QK_HEADS, QK_HEADS)
    c["t_begin"] = y * rows
    c["t_end"] = np.minimum(T, c["t_begin"] + rows)
    c["row0"] = c["bg"] * Tc
    wspan = rows // WAVES
    c["first"] = c["t_begin"] + w * wspan
    c["last"] = np.minimum(c["t_end"], c["first"] + wspan)
    return c


def replay_qk(bits, B, Hkv, G, Tc, T, D, cu=256):
    Hq, m, CB = Hkv * G, D // 128, 16 * bits
    G_, passes, pairs, chunks, tpg = qk_grid(bits, B, Hkv, T, m, Hq, cu)
    assert tpg % (WAVES * 16) == 0
    fast = m <= 2             # the batched path (one or two blocks per row)
    MD = m if fast else 1
    codes = Buf("k_codes", B * Hkv * Tc * m * CB)
    norms = Buf("k_norms", B * Hkv * Tc * m)
    q = Buf("q", B * Hq * D)
    scores = Buf("scores", B * Hq * T)
    c = wave_contexts(pairs, chunks, passes, Hkv, G, T, Tc, tpg)
    first, last, t_end, row0 = c["first"], c["last"], c["t_end"], c["row0"]
    b, h0, nh, wave = c["b"], c["h0"], c["nh"], c["wave"]
    ngroups = np.where(first < last, cdiv(last - first, 16), 0)
    nunits = ngroups * m
    kmax = int(rup(int(nunits.max()), QK_DEPTH)) + QK_DEPTH
    # query loads: the two preloaded head slots (D == 128), or every slice of every head
    for s in range(2):
        hh = wave + WAVES * s
        if m == 1:
            head = h0 + np.where(hh < nh, hh, 0)
            q.check((b * Hq + head) * 128 + LANE)
            q.check((b * Hq + head) * 128 + 64 + LANE)
        else:
            for j in range(m):
                base = (b * Hq + h0 + hh) * m * 128 + j * 128
                q.check(base + LANE, mask=hh < nh)
                q.check(base + 64 + LANE, mask=hh < nh)
    # code loads of every unit the loops may request (a superset: the loads clamp to the
    # wave's last row, so a wave never reads another wave's rows)
    lastc = np.where(first < last, last - 1, t_end - 1)
    own_lo = np.where(first < last, first, 0)
    for k in range(kmax):
        gi, j = k // m, k % m
        tb = np.minimum(first + gi * 16, lastc)
        r = np.minimum(N16, lastc - tb)
        assert np.all((tb + r <= lastc) & (tb + r >= own_lo)), "a load outside the wave's rows"
        blk0 = (row0 + tb) * m + j
        byte = blk0 * CB + r * m * CB + PART * 4 * bits
        codes.check(byte, width=4 * bits, align=4)
        if not fast:
            norms.check(blk0 + r * m)
    if fast:   # a batch's norms: one load per lane, clamped to the wave's last element
        emax = (row0 + lastc) * MD + (MD - 1)
        for k in range(0, kmax, QK_DEPTH):
            e0 = (row0 + first + 16 * (k // MD)) * MD
            norms.check(np.minimum(e0 + LANE, emax))
            assert np.all(emax < B * Hkv * Tc * m)
    # score stores
    if fast:
        rows16 = T % 4 == 0          # the tests' score buffers are 16-byte aligned
        sh, sr = LANE >> 3, 4 * (LANE & 7)
        rpb = 16 * QK_DEPTH // MD    # rows per batch
        nfull = np.where(rows16 & (first < last), (last - first) // rpb * QK_DEPTH, 0)
        shf = np.minimum(sh, nh - 1)
        # whole batches: a 16-byte score line per lane per pair of row groups
        for k0 in range(0, int(nfull.max()) if nfull.size else 0, QK_DEPTH):
            live = k0 < nfull
            for rg in range(1, QK_DEPTH // MD, 2):
                row = first + (k0 // MD + rg - 1) * 16 + sr
                assert np.all((row + 3 < last)[np.broadcast_to(live, row.shape)])
                scores.check((b * Hq + h0 + shf) * T + row, width=4, mask=live, align=4)
        # the ragged batch: the general loop, from nfull to the end of the units
        for k in range(0, kmax - QK_DEPTH):
            d = k % QK_DEPTH
            rg, jb = d // MD, d % MD
            if jb != MD - 1 or rg % 2 == 0:
                continue
            live = (k >= nfull) & (k < rup_arr(nunits, QK_DEPTH))
            if not live.any():
                continue
            t = first + (k // MD - 1) * 16 + sr
            ok = live & (sh < nh)
            vec = ok & rows16 & (t + 3 < last)
            scores.check((b * Hq + h0 + sh) * T + t, width=4, mask=vec, align=4)
            for i in range(4):
                el = ok & ~vec & (t + i < last)
                scores.check((b * Hq + h0 + sh) * T + t + i, mask=el)
        # LDS: the score stage (1 KB per wave)
        hu = 4 * (PART & 1) + (LANE >> 5)
        for rgp in range(2):
            assert ((hu + 2) * 32 + 16 * rgp + N16).max() < 256
        assert shf.max() * 32 + 4 * 7 + 3 < 256
    else:
        hu = 4 * (PART & 1) + (LANE >> 5)
        for k in range(int(nunits.max()) if nunits.size else 0):
            live = (k < rup_arr(nunits, QK_DEPTH)) & ((k % m) == m - 1)
            t = first + (k // m) * 16 + N16
            ok = live & (t < last)
            scores.check((b * Hq + h0 + hu) * T + t, mask=ok & (hu < nh))
            scores.check((b * Hq + h0 + hu + 2) * T + t, mask=ok & (hu + 2 < nh))
    return codes.n + norms.n + q.n + scores.n


def rup_arr(a, b):
    return -(-a // b) * b


# ---------------------------------------------------------------- decode attention

def attn_chunk_rows(bits, B, Hkv, T, Hq, M):
    G = Hq // Hkv
    passes = cdiv(G, QK_HEADS)
    step = WAVES * 16 * (4 // M)
    rnd = 256 * ATTN_GROUPS[(bits, 2 if G > QK_HEADS // 2 else 1, M)]
    rows = cdiv(T * B * Hkv * passes, rnd)
    rows = max(rows, cdiv(T, 65535))
    return max(rup(rows, step), step)


def replay_attn(bits, B, Hkv, G, Tc, T, D):
    Hq, M, CB = Hkv * G, D // 128, 16 * bits
    DEPTH, REC, RW = 4 // M, 4 + 128 * M, 4 * bits * M
    passes = cdiv(G, QK_HEADS)
    rows = attn_chunk_rows(bits, B, Hkv, T, Hq, M)
    chunks = cdiv(T, rows)
    assert chunks <= 65535 and rows % (WAVES * 16 * DEPTH) == 0
    kc = Buf("k_codes", B * Hkv * Tc * M * CB)
    vc = Buf("v_codes", B * Hkv * Tc * M * CB)
    kn = Buf("k_norms", B * Hkv * Tc * M)
    vn = Buf("v_norms", B * Hkv * Tc * M)
    q = Buf("q", B * Hq * D)
    work = Buf("workspace", B * Hq * chunks * REC)
    out = Buf("out", B * Hq * D)
    c = wave_contexts(B * Hkv * passes, chunks, passes, Hkv, G, T, Tc, rows)
    first, last, t_end, row0 = c["first"], c["last"], c["t_end"], c["row0"]
    b, h0, nh, wave, y = c["b"], c["h0"], c["nh"], c["wave"], c["y"]
    nunits = np.where(first < last, cdiv(last - first, 16), 0)
    lastc = np.where(nunits > 0, last - 1, t_end - 1)
    kmax = int(rup(int(nunits.max()), DEPTH)) + DEPTH
    for s in range(2):
        hh = wave + WAVES * s
        if M == 1:
            head = h0 + np.where(hh < nh, hh, 0)
            q.check((b * Hq + head) * 128 + LANE)
            q.check((b * Hq + head) * 128 + 64 + LANE)
        else:
            for j in range(M):
                base = (b * Hq + h0 + hh) * M * 128 + j * 128
                q.check(base + LANE, mask=hh < nh)
                q.check(base + 64 + LANE, mask=hh < nh)
    for k in range(kmax):
        tb = np.minimum(first + k * 16, lastc)
        r = np.minimum(N16, lastc - tb)
        for jb in range(M):
            byte = (row0 + tb) * M * CB + r * M * CB + jb * CB + PART * 4 * bits
            kc.check(byte, width=4 * bits, align=4)
            vc.check(byte, width=4 * bits, align=4)
    for k in range(0, kmax, DEPTH):
        tb = np.minimum(first + 16 * k, lastc)
        e = np.minimum(LANE, (lastc - tb) * M + (M - 1))
        kn.check((row0 + tb) * M + e)
        vn.check((row0 + tb) * M + e)
    # LDS tiles (words): a unit's code tile and a block's weight tile
    raw_words = 16 * RW + 4
    for j in range(2):
        for kb in range(2):
            row = (8 * kb + 2 * PART + j) * RW
            for jb in range(M):
                dA = (8 * bits * N16) >> 5
                assert (row + 4 * bits * jb + dA + 1).max() < raw_words
    assert (N16 * RW + 4 * bits * (M - 1) + PART * bits + bits - 1).max() < raw_words
    # the workspace records: thread t -> head t / 32, values 4 (t % 32) .. + 3
    tid = np.arange(256)
    h, v0 = tid >> 5, 4 * (tid & 31)
    xs, ys = np.meshgrid(np.arange(B * Hkv * passes), np.arange(chunks), indexing="ij")
    xs, ys = xs.reshape(-1, 1), ys.reshape(-1, 1)
    pas, bg = xs % passes, xs // passes
    bb, gg = bg // Hkv, bg % Hkv
    hh0 = gg * G + pas * QK_HEADS
    nnh = np.minimum(G - pas * QK_HEADS, QK_HEADS)
    rec = ((bb * Hq + hh0 + h) * chunks + ys) * REC
    for jb in range(M):
        work.check(rec + 4 + 128 * jb + v0, width=4, mask=h < nnh, align=4)
    work.check(rec, width=2, mask=(h < nnh) & (v0 == 0))
    # every (sequence, query head, chunk) record is written exactly once
    written = np.zeros(B * Hq * chunks, dtype=np.int64)
    sel = np.broadcast_to((h < nnh) & (v0 == 0), rec.shape)
    np.add.at(written, (rec[sel] // REC), 1)
    assert np.all(written == 1), "workspace records not written exactly once"
    # combine: one workgroup per (sequence, query head)
    bh = np.arange(B * Hq).reshape(-1, 1)
    for p in range(chunks):
        base = bh * chunks * REC + p * REC
        work.check(base)
        for jb in range(M):
            work.check(base + 4 + 128 * jb + LANE)
            work.check(base + 68 + 128 * jb + LANE)
    for jb in range(M):
        out.check(bh * 128 * M + 128 * jb + LANE)
        out.check(bh * 128 * M + 128 * jb + 64 + LANE)
    return kc.n + kn.n + q.n + work.n + out.n


# shapes (B, Hkv, G, Tc, T, D) of every q.K launch of the GPU tests, smoke, quality
# harness and benchmark
QK_SHAPES = [
    (2, 2, 4, 100, 97, 128), (1, 3, 1, 70, 70, 128), (2, 1, 8, 40, 33, 128), (1, 1, 12, 40, 40, 128),
    (1, 1, 16, 64, 61, 128), (1, 2, 3, 50, 50, 256), (1, 1, 2, 1100, 1100, 384), (1, 2, 5, 20, 17, 1024),
    (1, 1, 2, 24, 21, 2048), (1, 2, 4, 5000, 4999, 128), (1, 2, 4, 5000, 5000, 128),
    (1, 1, 12, 1000, 1000, 128), (2, 2, 4, 700, 644, 128),
    (1, 2, 4, 300, 300, 128), (1, 1, 3, 64, 64, 256),           # query magnitudes
    (2, 4, 4, 1000, 1000, 128),                                 # graph capture
    (1, 2, 4, 96, 96, 128),                                     # smoke
    (2, 8, 4, 4096, 4096, 128), (2, 8, 4, 32768, 32768, 128),   # quality harness
    (1, 8, 4, 32768, 32768, 128),                               # one layer
    (16, 8, 4, 32768, 32768, 128),                              # decode step
    (48, 8, 4, 32768, 32768, 128),                              # the 14B-shaped cache's keys
    (16, 8, 4, 32768, 32768, 256), (32, 4, 4, 32768, 32768, 256),   # head_dim 256
]

ATTN_SHAPES = [
    (1, 2, 4, 100, 97, 128), (2, 1, 8, 40, 33, 128), (1, 1, 12, 300, 300, 128), (1, 3, 1, 70, 70, 128),
    (1, 2, 2, 1, 1, 128), (1, 2, 4, 5000, 4999, 128), (3, 2, 4, 2000, 1500, 128),
    (1, 2, 4, 100, 97, 256), (2, 1, 8, 40, 33, 256), (1, 1, 12, 300, 300, 256), (1, 3, 1, 70, 70, 256),
    (1, 2, 2, 1, 1, 256), (1, 2, 4, 5000, 4999, 256), (3, 2, 4, 2000, 1500, 256),
    (1, 1, 16, 64, 61, 128), (1, 2, 3, 50, 50, 128), (2, 2, 5, 300, 257, 128),   # groups 16, 3, 5
    (1, 1, 16, 64, 61, 256), (1, 2, 3, 50, 50, 256), (2, 2, 5, 300, 257, 256),
    (1, 2, 4, 600, 600, 128), (1, 2, 4, 600, 590, 128), (1, 2, 4, 300, 300, 128),     # extremes
    (1, 2, 4, 600, 600, 256), (1, 2, 4, 600, 590, 256), (1, 2, 4, 300, 300, 256),
    (2, 2, 4, 3000, 3000, 128),                                 # side stream
    (4, 8, 4, 8192, 8192, 128), (4, 8, 4, 8192, 8192, 256), (2, 2, 4, 1200, 1000, 128),  # no-alloc
    (1, 2, 4, 3000, 2999, 256),                                 # rotation
    (2, 4, 4, 1000, 999, 128),                                  # graph capture
    (1, 2, 4, 96, 96, 128),                                     # smoke
    (2, 8, 4, 4096, 4096, 128), (2, 8, 4, 32768, 32768, 128),   # quality harness
    (16, 8, 4, 32768, 32768, 128),                              # decode step
    (16, 8, 4, 32768, 32768, 256), (32, 4, 4, 32768, 32768, 256),   # head_dim 256
]


@pytest.mark.parametrize("shape", QK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_qk_kernel_accesses_stay_in_bounds(shape):
    for bits in (3, 2):
        for cu in (256, 304, 80):   # the grid follows the device's compute units
            assert replay_qk(bits, *shape, cu=cu) > 0


@pytest.mark.parametrize("shape", ATTN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_attention_kernels_accesses_stay_in_bounds(shape):
    for bits in (3, 2):
        assert replay_attn(bits, *shape) > 0


def test_replay_catches_the_unclamped_head_store():
    """The replay is not vacuous: without the clamp of a pass's heads (the q.K store that
    once faulted), a pass of four heads would write score lines past its sequence's rows;
    restated for group 12 (passes of eight and four heads), the last sequence's second
    pass reaches past the end of the buffer."""
    B, Hkv, G, T = 1, 1, 12, 40
    Hq = Hkv * G
    G_, passes, pairs, chunks, tpg = qk_grid(3, B, Hkv, T, 1, Hq, 256)
    c = wave_contexts(pairs, chunks, passes, Hkv, G, T, T, tpg)
    sh = LANE >> 3
    head = c["h0"] + sh                      # the unclamped head of each score lane
    assert (head >= Hq).any()                # the second pass's lanes past head 11
    assert ((head * T).max() + T) > B * Hq * T


# ---------------------------------------------------------------- encoder tile order

def encoder_tiles(bits, nblocks, grid, tile_blocks=32):
    """The tiles each wave of encode_kernel takes, restated: wave w of workgroup x starts
    at tile 4 x + w, which turbo2 remaps inside each whole run of 32 tiles when the grid
    gives every wave one tile, then steps by the grid's wave count."""
    ntiles = cdiv(nblocks, tile_blocks)
    stride = grid * WAVES
    taken = []
    for x in range(grid):
        for w in range(WAVES):
            t = x * WAVES + w
            if bits == 2 and stride >= ntiles and (t | 31) < ntiles:
                t = (t & ~31) + w * 8 + (x & 7)
            while t < ntiles:
                taken.append(t)
                t += stride
    return ntiles, taken


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("nblocks", [1, 31, 32, 33, 1000, 1024, 1056, 131136, 25165824 // 64])
def test_encoder_takes_every_tile_once(bits, nblocks):
    """One tile per wave (the default grid) and a grid capped at one or two workgroups per
    CU: every tile of the input is encoded exactly once, whatever the order."""
    ntiles = cdiv(nblocks, 32)
    for grid in (cdiv(ntiles, WAVES), min(cdiv(ntiles, WAVES), 256), min(cdiv(ntiles, WAVES), 512)):
        n, taken = encoder_tiles(bits, nblocks, grid)
        assert sorted(taken) == list(range(n)), (bits, nblocks, grid)


def test_encoder_tile_order_matches_the_kernel():
    src = open(KERNELS).read()
    assert "if (gridDim.x * kWavesPerGroup >= ntiles && (tile | 31u) < ntiles)" in src
    assert "tile = (tile & ~31u) + wave * 8u + (blockIdx.x & 7u);" in src
    assert "uint32_t tile = blockIdx.x * kWavesPerGroup + wave;" in src
