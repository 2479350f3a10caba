"""Python binding of libtq, the MI355X (gfx950) turbo3 / turbo2 KV-cache block codec.

Argument marshalling only: every function forwards torch device pointers, sizes
and the current HIP stream to the C ABI declared in ``include/tq.h``; all
computation happens in the library's HIP kernels.  There is no CPU fallback:
tensors must live on the GPU, and a missing ``libtq.so`` raises at import of
the first call.

Layouts (the library's block format):
  x       fp16 [L, H, T, D], D = 128 * m, contiguous
  codes   uint8 [L, H, Tc, m, 16 * type]   (type = 3 turbo3, 2 turbo2)
  norms   fp16 [L, H, Tc, m]
  q       fp16 [B, Hq, D];  scores fp32 [B, Hq, T]
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

__all__ = [
    "TQ_TURBO2", "TQ_TURBO3", "TQError", "lib", "lib_path", "header_functions",
    "tq_block_code_bytes", "tq_block_bytes", "tq_codes_nbytes", "tq_norms_count",
    "tq_status_string", "tq_codebook", "tq_encode", "tq_decode", "tq_qk_scores",
    "tq_attn_workspace_bytes", "tq_attn_decode", "tq_attn_decode_noalloc", "TQ_ATTN_SCRATCH_BYTES",
    "tq_pack_records", "tq_unpack_records",
    "tq_time_next_launch", "sign_words", "empty_cache",
]

TQ_TURBO2 = 2
TQ_TURBO3 = 3
TQ_ATTN_SCRATCH_BYTES = 8 << 20   # the static workspace of tq_attn_decode_noalloc

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libtq.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "tq.h")

STATUS = {0: "TQ_OK", -1: "TQ_ERR_TYPE", -2: "TQ_ERR_SHAPE", -3: "TQ_ERR_RANGE",
          -4: "TQ_ERR_NULL", -5: "TQ_ERR_ALIGN", -6: "TQ_ERR_ALIAS", -7: "TQ_ERR_DEVICE",
          -8: "TQ_ERR_WORKSPACE"}


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {tq_status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing; build it with "
                           "`python -m kv_cache_quantization_block_amd.build`")
    check_build()
    L = ctypes.CDLL(lib_path)
    i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    L.tq_block_code_bytes.restype = i32
    L.tq_block_code_bytes.argtypes = [i32]
    L.tq_block_bytes.restype = i32
    L.tq_block_bytes.argtypes = [i32]
    L.tq_codes_nbytes.restype = i64
    L.tq_codes_nbytes.argtypes = [i32, i64, i64, i64, i64]
    L.tq_norms_count.restype = i64
    L.tq_norms_count.argtypes = [i64, i64, i64, i64]
    L.tq_status_string.restype = ctypes.c_char_p
    L.tq_status_string.argtypes = [i32]
    L.tq_codebook.restype = i32
    L.tq_codebook.argtypes = [i32, vp, vp]
    L.tq_encode.restype = i32
    L.tq_encode.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp]
    L.tq_decode.restype = i32
    L.tq_decode.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp]
    L.tq_qk_scores.restype = i32
    L.tq_qk_scores.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64, vp, i64, f32, vp, vp]
    L.tq_attn_workspace_bytes.restype = i64
    L.tq_attn_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64]
    L.tq_attn_decode.restype = i32
    L.tq_attn_decode.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, f32, vp,
                                 vp, i64, vp]
    L.tq_attn_decode_noalloc.restype = i32
    L.tq_attn_decode_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64,
                                         f32, vp, vp]
    L.tq_pack_records.restype = i32
    L.tq_pack_records.argtypes = [i32, vp, vp, i64, vp, vp]
    L.tq_unpack_records.restype = i32
    L.tq_unpack_records.argtypes = [i32, vp, i64, vp, vp, vp]
    L.tq_time_next_launch.restype = i32
    L.tq_time_next_launch.argtypes = [vp, vp]
    for name, plain in (("tq_encode_rot", L.tq_encode), ("tq_decode_rot", L.tq_decode),
                        ("tq_qk_scores_rot", L.tq_qk_scores), ("tq_attn_decode_rot", L.tq_attn_decode)):
        f = getattr(L, name)
        f.restype = i32
        f.argtypes = [i32, vp] + plain.argtypes[1:]
    _lib = L
    return L


def check_build() -> None:
    """Raise unless libtq.so was built from the sources now in the tree: the build
    writes the sha256 of its sources beside the library (libtq.so.srcsha)."""
    from . import build as _build
    try:
        built = open(_build.SRC_SHA).read().strip()
    except OSError:
        raise RuntimeError(f"{_build.SRC_SHA} is missing: rebuild libtq.so with "
                           "`python -m kv_cache_quantization_block_amd.build`") from None
    if built != _build.source_sha():
        raise RuntimeError("libtq.so was built from other sources than those in "
                           f"{_build.CSRC} and include/; rebuild it with "
                           "`python -m kv_cache_quantization_block_amd.build`")


def header_functions() -> list[str]:
    """Names of the functions include/tq.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)


def tq_block_code_bytes(type: int) -> int:
    return lib().tq_block_code_bytes(type)


def tq_block_bytes(type: int) -> int:
    return lib().tq_block_bytes(type)


def tq_codes_nbytes(type: int, L: int, H: int, Tc: int, D: int) -> int:
    return lib().tq_codes_nbytes(type, L, H, Tc, D)


def tq_norms_count(L: int, H: int, Tc: int, D: int) -> int:
    return lib().tq_norms_count(L, H, Tc, D)


def tq_status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def tq_codebook(type: int):
    """(levels, thresholds) float32 lists the kernels use."""
    n = 1 << type
    lv = (ctypes.c_float * n)()
    th = (ctypes.c_float * (n - 1))()
    rc = lib().tq_codebook(type, ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p))
    if rc:
        raise TQError(rc, "tq_codebook")
    return list(lv), list(th)


# ---------------------------------------------------------------- tensor calls

def sign_words(signs):
    """128 diagonal entries of the randomised rotation H D (+1 / -1, or bools where True
    means -1) -> the four 32-bit words the _rot calls take (bit p set <=> D_pp = -1).
    Words made by an earlier call pass through unchanged, so a caller that launches
    often can convert its signs once."""
    if isinstance(signs, ctypes.Array) and signs._type_ is ctypes.c_uint32 and len(signs) == 4:
        return signs
    if isinstance(signs, torch.Tensor):
        signs = signs.detach().cpu().numpy()
    v = np.asarray(signs)
    if v.shape != (128,):
        raise ValueError("signs must hold 128 entries")
    if v.dtype == np.bool_:
        neg = v
    else:
        if not np.all(np.abs(v.astype(np.float64)) == 1.0):
            raise ValueError("signs must be +1 / -1 (or bools)")
        neg = v.astype(np.float64) < 0
    w = [int(np.sum(neg[32 * k:32 * k + 32].astype(np.uint64) << np.arange(32, dtype=np.uint64)))
         for k in range(4)]
    return (ctypes.c_uint32 * 4)(*w)


def _stream(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    if s.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {s.device}, not the current device "
                         f"cuda:{torch.cuda.current_device()}")
    return s.cuda_stream or None


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    """Device pointer of t, which must be a contiguous tensor of `dtype` on the current
    device (the library launches on the current device)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not the current device "
                         f"cuda:{torch.cuda.current_device()} (use torch.cuda.device)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def empty_cache(type: int, L: int, H: int, Tc: int, D: int, device="cuda"):
    """Uninitialised (codes, norms) planes of a [L, H, Tc, D] cache."""
    if D % 128:
        raise ValueError("D must be a multiple of 128")
    m = D // 128
    codes = torch.empty((L, H, Tc, m, 16 * type), dtype=torch.uint8, device=device)
    norms = torch.empty((L, H, Tc, m), dtype=torch.float16, device=device)
    return codes, norms


def _cache_dims(codes: torch.Tensor, norms: torch.Tensor, type: int):
    if codes.dim() != 5 or codes.shape[4] != 16 * type:
        raise ValueError(f"codes must be [L, H, Tc, D/128, {16 * type}]")
    L, H, Tc, m, _ = codes.shape
    if tuple(norms.shape) != (L, H, Tc, m):
        raise ValueError("norms must be [L, H, Tc, D/128]")
    return L, H, Tc, m * 128


def tq_encode(type: int, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
              t0: int = 0, stream=None, signs=None) -> None:
    """Encode x [L, H, T, D] into cache rows [t0, t0 + T) (asynchronous).  signs: None
    (rotation H) or the 128 signs of the randomised rotation H D (tq_encode_rot)."""
    L, H, Tc, D = _cache_dims(codes, norms, type)
    if x.dim() != 4 or tuple(x.shape[:2]) != (L, H) or x.shape[3] != D:
        raise ValueError("x must be [L, H, T, D] matching the cache")
    T = x.shape[2]
    args = (_dev(x, "x", torch.float16), L, H, T, D, _dev(codes, "codes", torch.uint8),
            _dev(norms, "norms", torch.float16), Tc, t0, _stream(stream))
    rc = lib().tq_encode(type, *args) if signs is None else lib().tq_encode_rot(type, sign_words(signs), *args)
    if rc:
        raise TQError(rc, "tq_encode")


def tq_decode(type: int, codes: torch.Tensor, norms: torch.Tensor, t0: int, x: torch.Tensor,
              stream=None, signs=None) -> None:
    """Decode cache rows [t0, t0 + T) into x [L, H, T, D] fp16 (asynchronous).  signs: as
    the cache was encoded with (tq_decode_rot), or None."""
    L, H, Tc, D = _cache_dims(codes, norms, type)
    if x.dim() != 4 or tuple(x.shape[:2]) != (L, H) or x.shape[3] != D:
        raise ValueError("x must be [L, H, T, D] matching the cache")
    T = x.shape[2]
    args = (_dev(codes, "codes", torch.uint8), _dev(norms, "norms", torch.float16),
            L, H, Tc, D, t0, T, _dev(x, "x", torch.float16), _stream(stream))
    rc = lib().tq_decode(type, *args) if signs is None else lib().tq_decode_rot(type, sign_words(signs), *args)
    if rc:
        raise TQError(rc, "tq_decode")


def tq_qk_scores(type: int, k_codes: torch.Tensor, k_norms: torch.Tensor, q: torch.Tensor,
                 scale: float, scores: torch.Tensor, stream=None, signs=None) -> None:
    """scores [B, Hq, T] = scale * q . k_hat over key-cache rows [0, T) (asynchronous).
    signs: as the cache was encoded with (tq_qk_scores_rot), or None."""
    B, Hkv, Tc, D = _cache_dims(k_codes, k_norms, type)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, Hq, D] matching the cache")
    Hq = q.shape[1]
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (B, Hq):
        raise ValueError("scores must be [B, Hq, T]")
    T = scores.shape[2]
    args = (_dev(k_codes, "k_codes", torch.uint8), _dev(k_norms, "k_norms", torch.float16), B,
            Hkv, Tc, D, T, _dev(q, "q", torch.float16), Hq, float(scale),
            _dev(scores, "scores", torch.float32), _stream(stream))
    rc = (lib().tq_qk_scores(type, *args) if signs is None
          else lib().tq_qk_scores_rot(type, sign_words(signs), *args))
    if rc:
        raise TQError(rc, "tq_qk_scores")


def tq_attn_workspace_bytes(type: int, B: int, Hkv: int, Tc: int, D: int, T: int, Hq: int) -> int:
    """Device workspace bytes tq_attn_decode needs for these sizes."""
    r = lib().tq_attn_workspace_bytes(type, B, Hkv, Tc, D, T, Hq)
    if r < 0:
        raise TQError(int(r), "tq_attn_workspace_bytes")
    return int(r)


def tq_attn_decode(type: int, k_codes: torch.Tensor, k_norms: torch.Tensor, v_codes: torch.Tensor,
                   v_norms: torch.Tensor, q: torch.Tensor, scale: float, out: torch.Tensor,
                   T: int | None = None, workspace: torch.Tensor | None = None, stream=None,
                   signs=None) -> None:
    """out [B, Hq, D] (fp32) = softmax over rows [0, T) of scale * q . k_hat, applied to v_hat
    (asynchronous).  workspace: a uint8 device tensor of at least tq_attn_workspace_bytes;
    when None, one is allocated here with torch (the library itself never allocates).
    signs: as the caches were encoded with (tq_attn_decode_rot), or None."""
    B, Hkv, Tc, D = _cache_dims(k_codes, k_norms, type)
    if _cache_dims(v_codes, v_norms, type) != (B, Hkv, Tc, D):
        raise ValueError("K and V caches must have the same shape")
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, Hq, D] matching the cache")
    Hq = q.shape[1]
    if out.dim() != 3 or tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    T = Tc if T is None else int(T)
    need = tq_attn_workspace_bytes(type, B, Hkv, Tc, D, T, Hq)
    if workspace is None:
        # allocated on the stream the kernels run on: the caching allocator hands these
        # bytes to another allocation only once that stream's work is done with them
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=out.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-d uint8 tensor")
    args = (_dev(k_codes, "k_codes", torch.uint8), _dev(k_norms, "k_norms", torch.float16),
            _dev(v_codes, "v_codes", torch.uint8), _dev(v_norms, "v_norms", torch.float16), B, Hkv,
            Tc, D, T, _dev(q, "q", torch.float16), Hq, float(scale),
            _dev(out, "out", torch.float32), _dev(workspace, "workspace", torch.uint8),
            workspace.numel(), _stream(stream))
    rc = (lib().tq_attn_decode(type, *args) if signs is None
          else lib().tq_attn_decode_rot(type, sign_words(signs), *args))
    if rc:
        raise TQError(rc, "tq_attn_decode")


def tq_attn_decode_noalloc(type: int, k_codes: torch.Tensor, k_norms: torch.Tensor,
                           v_codes: torch.Tensor, v_norms: torch.Tensor, q: torch.Tensor,
                           scale: float, out: torch.Tensor, T: int | None = None, stream=None,
                           signs=None) -> None:
    """tq_attn_decode without a workspace: the library's static device scratch array
    (TQ_ATTN_SCRATCH_BYTES per device) takes its place, and nothing is allocated.
    Calls that overlap on one device race on that array."""
    B, Hkv, Tc, D = _cache_dims(k_codes, k_norms, type)
    if _cache_dims(v_codes, v_norms, type) != (B, Hkv, Tc, D):
        raise ValueError("K and V caches must have the same shape")
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, Hq, D] matching the cache")
    Hq = q.shape[1]
    if out.dim() != 3 or tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    T = Tc if T is None else int(T)
    rc = lib().tq_attn_decode_noalloc(
        type, None if signs is None else sign_words(signs),
        _dev(k_codes, "k_codes", torch.uint8), _dev(k_norms, "k_norms", torch.float16),
        _dev(v_codes, "v_codes", torch.uint8), _dev(v_norms, "v_norms", torch.float16), B, Hkv,
        Tc, D, T, _dev(q, "q", torch.float16), Hq, float(scale), _dev(out, "out", torch.float32),
        _stream(stream))
    if rc:
        raise TQError(rc, "tq_attn_decode_noalloc")


def _record_args(type: int, codes: torch.Tensor, norms: torch.Tensor, records: torch.Tensor):
    nb = norms.numel()
    if codes.numel() != nb * 16 * type or records.numel() != nb * (2 + 16 * type):
        raise ValueError("codes / norms / records sizes do not describe the same blocks")
    return nb


def tq_pack_records(type: int, codes: torch.Tensor, norms: torch.Tensor, records: torch.Tensor,
                    stream=None) -> None:
    """Both planes (any shape, contiguous) -> interleaved records, a uint8 tensor of
    norms.numel() * (2 + 16 * type) bytes (asynchronous)."""
    nb = _record_args(type, codes, norms, records)
    rc = lib().tq_pack_records(type, _dev(codes, "codes", torch.uint8), _dev(norms, "norms", torch.float16),
                               nb, _dev(records, "records", torch.uint8), _stream(stream))
    if rc:
        raise TQError(rc, "tq_pack_records")


def _event_handle(e):
    if e is None:
        return None
    if isinstance(e, int):
        return e
    h = getattr(e, "cuda_event", 0)      # torch.cuda.Event: its hipEvent_t, once created
    if not h:
        raise ValueError("the event has no HIP event yet: record it once first "
                         "(torch.cuda.Event creates its event at the first record)")
    return h


def tq_time_next_launch(start_event, stop_event) -> None:
    """Arm the per-thread timing hook: the next kernel launched by a tq_* call records
    its own start / stop on these events (torch.cuda.Event with timing, already
    recorded once; raw hipEvent_t ints; or None)."""
    rc = lib().tq_time_next_launch(_event_handle(start_event), _event_handle(stop_event))
    if rc:
        raise TQError(rc, "tq_time_next_launch")


def tq_unpack_records(type: int, records: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
                      stream=None) -> None:
    """Interleaved records -> both planes (asynchronous)."""
    nb = _record_args(type, codes, norms, records)
    rc = lib().tq_unpack_records(type, _dev(records, "records", torch.uint8), nb,
                                 _dev(codes, "codes", torch.uint8), _dev(norms, "norms", torch.float16),
                                 _stream(stream))
    if rc:
        raise TQError(rc, "tq_unpack_records")
