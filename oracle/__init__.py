"""CPU oracle of the turbo3 / turbo2 KV-cache block codec (binary64, plain C).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (``kv_cache_quantization_block_amd``) and imports nothing
from it; the product path never imports this.

The C source (``tq_oracle.c``) follows the TurboQuant turbo3/turbo2 article
(openalchemy.io, "llama.cpp に TurboQuant を実装"): sections
"TurboQuant の何が違うのか" (rotate, Lloyd-Max, FWHT), "どこまで小さくなるのか"
(128 values + one FP16 norm per block) and "実モデルでの数値" (head_dim = 128*m).

Arrays are numpy; fp16 tensors are passed as ``np.float16`` (bit patterns are
what crosses into C).  Every function validates shapes and raises ValueError.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtqoracle.so")
BLOCK = 128

# gcc: IEEE semantics only -- no -ffast-math, no FMA contraction.
BUILD_CMD = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
             "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> str:
    """Compile the oracle shared library in place; returns its path."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.tqo_half_to_double.restype = dbl
    lib.tqo_half_to_double.argtypes = [ctypes.c_uint16]
    lib.tqo_double_to_half.restype = ctypes.c_uint16
    lib.tqo_double_to_half.argtypes = [dbl]
    lib.tqo_codebook.restype = i32
    lib.tqo_codebook.argtypes = [i32, vp, vp]
    lib.tqo_fwht128.restype = None
    lib.tqo_fwht128.argtypes = [vp]
    lib.tqo_encode_blocks.restype = i32
    lib.tqo_encode_blocks.argtypes = [i32, vp, i64, vp, vp, vp, vp, i32]
    lib.tqo_decode_blocks.restype = i32
    lib.tqo_decode_blocks.argtypes = [i32, vp, vp, i64, vp, vp, vp, i32]
    lib.tqo_encode.restype = i32
    lib.tqo_encode.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp, i32]
    lib.tqo_decode.restype = i32
    lib.tqo_decode.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, vp, i32]
    lib.tqo_qk.restype = i32
    lib.tqo_qk.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64, vp, i64, dbl, vp, vp, i32]
    lib.tqo_attn_decode.restype = i32
    lib.tqo_attn_decode.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, dbl,
                                    vp, vp, i32]
    lib.tqo_pack_records.restype = i32
    lib.tqo_pack_records.argtypes = [i32, vp, vp, i64, vp]
    lib.tqo_unpack_records.restype = i32
    lib.tqo_unpack_records.argtypes = [i32, vp, i64, vp, vp]
    _lib = lib
    return lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise ValueError(f"expected float16, got {a.dtype}")
    return a


def _signs(signs):
    """None, or the 128 diagonal entries (+1 / -1) of the randomised rotation H D."""
    if signs is None:
        return None
    d = np.ascontiguousarray(signs, dtype=np.float64).reshape(-1)
    if d.shape != (BLOCK,) or not np.all(np.abs(d) == 1.0):
        raise ValueError("signs must be 128 values of +1 / -1")
    return d


def _check_bits(bits):
    if bits not in (2, 3):
        raise ValueError("bits must be 2 (turbo2) or 3 (turbo3)")


def code_bytes(bits: int) -> int:
    """Bytes of packed codes per 128-value block (16 * bits)."""
    return 16 * bits


def half_to_double(h: int) -> float:
    return _load().tqo_half_to_double(int(h) & 0xFFFF)


def double_to_half_bits(x: float) -> int:
    return int(_load().tqo_double_to_half(float(x)))


def codebook(bits: int):
    """(levels[2^bits], thresholds[2^bits - 1], iterations) of the N(0,1) Lloyd-Max quantiser."""
    L = 1 << bits
    lv = np.zeros(L, np.float64)
    th = np.zeros(L - 1, np.float64)
    it = _load().tqo_codebook(bits, _ptr(lv), _ptr(th))
    if it < 0:
        raise ValueError("codebook solver failed")
    return lv, th, it


def fwht128(v) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard transform of each 128-row of v (float64 copy)."""
    v = np.array(v, dtype=np.float64, copy=True).reshape(-1, BLOCK)
    lib = _load()
    for r in range(v.shape[0]):
        row = np.ascontiguousarray(v[r])
        lib.tqo_fwht128(_ptr(row))
        v[r] = row
    return v


def encode_blocks(bits: int, x, nthreads: int | None = None, want_dist: bool = False,
                  signs=None):
    """x: fp16 [..., 128] → (codes u8 [nb, 16*bits], norms fp16 [nb], dist f64 [nb,128] | None).
    signs: None (H) or 128 values +-1 (the randomised rotation H D)."""
    _check_bits(bits)
    d = _signs(signs)
    x = _c16(x).reshape(-1, BLOCK)
    nb = x.shape[0]
    codes = np.zeros((nb, code_bytes(bits)), np.uint8)
    norms = np.zeros(nb, np.float16)
    dist = np.zeros((nb, BLOCK), np.float64) if want_dist else None
    rc = _load().tqo_encode_blocks(bits, _ptr(x), nb, _ptr(codes), _ptr(norms), _ptr(dist),
                                   _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_encode_blocks failed")
    return codes, norms, dist


def decode_blocks(bits: int, codes, norms, nthreads: int | None = None, signs=None):
    """codes u8 [nb, 16*bits], norms fp16 [nb] → (xhat f64 [nb,128], fp16 RNE of it)."""
    _check_bits(bits)
    d = _signs(signs)
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, code_bytes(bits))
    norms = _c16(norms).reshape(-1)
    nb = codes.shape[0]
    if norms.shape[0] != nb:
        raise ValueError("codes / norms block counts differ")
    xhat = np.zeros((nb, BLOCK), np.float64)
    x16 = np.zeros((nb, BLOCK), np.float16)
    rc = _load().tqo_decode_blocks(bits, _ptr(codes), _ptr(norms), nb, _ptr(xhat), _ptr(x16),
                                   _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_decode_blocks failed")
    return xhat, x16


def encode(bits: int, x, codes, norms, t0: int = 0, nthreads: int | None = None,
           want_dist: bool = False, signs=None):
    """x fp16 [L,H,T,D] → writes cache rows [t0, t0+T) of codes u8 [L,H,Tc,D/128,16*bits]
    and norms fp16 [L,H,Tc,D/128] in place.  Returns dist [L,H,T,D] (or None)."""
    _check_bits(bits)
    d = _signs(signs)
    x = _c16(x)
    L, H, T, D = x.shape
    if D % BLOCK:
        raise ValueError("D must be a multiple of 128")
    m = D // BLOCK
    Tc = codes.shape[2]
    if codes.shape != (L, H, Tc, m, code_bytes(bits)) or codes.dtype != np.uint8 \
            or not codes.flags.c_contiguous:
        raise ValueError("bad codes array")
    if norms.shape != (L, H, Tc, m) or norms.dtype != np.float16 or not norms.flags.c_contiguous:
        raise ValueError("bad norms array")
    dist = np.zeros((L, H, T, D), np.float64) if want_dist else None
    rc = _load().tqo_encode(bits, _ptr(x), L, H, T, D, _ptr(codes), _ptr(norms), Tc, t0,
                            _ptr(dist), _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_encode failed")
    return dist


def decode(bits: int, codes, norms, t0: int, T: int, nthreads: int | None = None, signs=None):
    """Cache rows [t0, t0+T) → (xhat f64 [L,H,T,D], fp16 RNE of it)."""
    _check_bits(bits)
    d = _signs(signs)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    norms = _c16(norms)
    L, H, Tc, m, cb = codes.shape
    if cb != code_bytes(bits) or norms.shape != (L, H, Tc, m):
        raise ValueError("bad cache arrays")
    D = m * BLOCK
    xhat = np.zeros((L, H, T, D), np.float64)
    x16 = np.zeros((L, H, T, D), np.float16)
    rc = _load().tqo_decode(bits, _ptr(codes), _ptr(norms), L, H, Tc, D, t0, T, _ptr(xhat),
                            _ptr(x16), _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_decode failed")
    return xhat, x16


def qk_scores(bits: int, k_codes, k_norms, q, scale: float, T: int | None = None,
              nthreads: int | None = None, signs=None):
    """K cache [B,Hkv,Tc,D/128,...] + q fp16 [B,Hq,D] → scores f64 [B,Hq,T]."""
    _check_bits(bits)
    d = _signs(signs)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    k_norms = _c16(k_norms)
    q = _c16(q)
    B, Hkv, Tc, m, cb = k_codes.shape
    Bq, Hq, D = q.shape
    if cb != code_bytes(bits) or k_norms.shape != (B, Hkv, Tc, m) or Bq != B or D != m * BLOCK:
        raise ValueError("bad q / cache arrays")
    T = Tc if T is None else T
    scores = np.zeros((B, Hq, T), np.float64)
    rc = _load().tqo_qk(bits, _ptr(k_codes), _ptr(k_norms), B, Hkv, Tc, D, T, _ptr(q), Hq,
                        float(scale), _ptr(scores), _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_qk failed")
    return scores


def attn_decode(bits: int, k_codes, k_norms, v_codes, v_norms, q, scale: float,
                T: int | None = None, nthreads: int | None = None, signs=None):
    """K and V caches [B,Hkv,Tc,D/128,...] + q fp16 [B,Hq,D] → out f64 [B,Hq,D]:
    softmax over rows [0, T) of scale * q.k_hat, applied to v_hat."""
    _check_bits(bits)
    d = _signs(signs)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    k_norms, v_norms, q = _c16(k_norms), _c16(v_norms), _c16(q)
    B, Hkv, Tc, m, cb = k_codes.shape
    Bq, Hq, D = q.shape
    if (cb != code_bytes(bits) or v_codes.shape != k_codes.shape or k_norms.shape != (B, Hkv, Tc, m)
            or v_norms.shape != k_norms.shape or Bq != B or D != m * BLOCK):
        raise ValueError("bad q / cache arrays")
    T = Tc if T is None else T
    out = np.zeros((B, Hq, D), np.float64)
    rc = _load().tqo_attn_decode(bits, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
                                 B, Hkv, Tc, D, T, _ptr(q), Hq, float(scale), _ptr(out),
                                 _ptr(d), nthreads or default_threads())
    if rc:
        raise ValueError("tqo_attn_decode failed")
    return out


def pack_records(bits: int, codes, norms) -> np.ndarray:
    """codes u8 [..., 16*bits] + norms fp16 [...] → records u8 [nb, 2 + 16*bits]."""
    _check_bits(bits)
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, code_bytes(bits))
    norms = _c16(norms).reshape(-1)
    nb = codes.shape[0]
    if norms.shape[0] != nb:
        raise ValueError("codes / norms block counts differ")
    rec = np.zeros((nb, 2 + code_bytes(bits)), np.uint8)
    if _load().tqo_pack_records(bits, _ptr(codes), _ptr(norms), nb, _ptr(rec)):
        raise ValueError("tqo_pack_records failed")
    return rec


def unpack_records(bits: int, records):
    """records u8 [nb, 2 + 16*bits] → (codes u8 [nb, 16*bits], norms fp16 [nb])."""
    _check_bits(bits)
    rec = np.ascontiguousarray(records, dtype=np.uint8).reshape(-1, 2 + code_bytes(bits))
    nb = rec.shape[0]
    codes = np.zeros((nb, code_bytes(bits)), np.uint8)
    norms = np.zeros(nb, np.float16)
    if _load().tqo_unpack_records(bits, _ptr(rec), nb, _ptr(codes), _ptr(norms)):
        raise ValueError("tqo_unpack_records failed")
    return codes, norms
