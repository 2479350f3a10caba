"""The C-ABI library on the CPU: it loads, exports every declared symbol, sizes
its planes as the article prints, rejects bad arguments before touching HIP,
and carries float32 codebooks equal to the oracle's binary64 solution rounded
to float.  No compute call runs here (no GPU)."""
import ctypes
import os

import numpy as np
import pytest

import kv_cache_quantization_block_amd as tq
import oracle

OK, E_TYPE, E_SHAPE, E_RANGE, E_NULL, E_ALIGN, E_ALIAS = 0, -1, -2, -3, -4, -5, -6
E_WORKSPACE = -8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tq.lib_path):
        from kv_cache_quantization_block_amd import build
        build.build()
    return tq.lib()


def test_exports_every_declared_symbol(L):
    names = tq.header_functions()
    assert {"tq_encode", "tq_decode", "tq_qk_scores", "tq_codebook", "tq_attn_decode",
            "tq_attn_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_binding_covers_every_declared_call():
    """Each declared call has a Python function of the same name (the _rot calls are
    the plain functions' signs= argument), and every name the binding exports exists."""
    for n in tq.header_functions():
        plain = n[:-4] if n.endswith("_rot") else n
        assert callable(getattr(tq, plain, None)), plain
    for n in tq.__all__:
        assert hasattr(tq, n), n


def test_sizes():
    """Section "どこまで小さくなるのか": 128 values + one fp16 norm = 50 / 34 bytes."""
    assert tq.tq_block_code_bytes(3) == 48 and tq.tq_block_bytes(3) == 50
    assert tq.tq_block_code_bytes(2) == 32 and tq.tq_block_bytes(2) == 34
    assert tq.tq_block_bytes(4) == E_TYPE and tq.tq_block_code_bytes(1) == E_TYPE
    assert tq.tq_codes_nbytes(3, 48, 8, 32768, 128) == 48 * 8 * 32768 * 48
    assert tq.tq_codes_nbytes(2, 32, 4, 32768, 256) == 32 * 4 * 32768 * 2 * 32
    assert tq.tq_norms_count(32, 4, 32768, 256) == 32 * 4 * 32768 * 2
    assert tq.tq_codes_nbytes(3, 1, 1, 1, 100) == E_SHAPE
    assert tq.tq_norms_count(1, 1, 1, 0) == E_SHAPE
    assert tq.tq_codes_nbytes(3, 1 << 40, 1 << 40, 1, 128) == E_SHAPE   # overflow


def test_status_strings():
    for code, name in tq.STATUS.items():
        assert tq.tq_status_string(code).startswith(name)
    assert "unknown" in tq.tq_status_string(12345)


@pytest.mark.parametrize("bits", [2, 3])
def test_codebook_is_oracle_solution_rounded_to_float(bits):
    """The library solves the Lloyd-Max conditions on its own; its float32 levels and
    thresholds must equal float32(oracle's binary64 solution)."""
    lv, th = tq.tq_codebook(bits)
    olv, oth, _ = oracle.codebook(bits)
    assert np.array_equal(np.array(lv, np.float32), olv.astype(np.float32))
    assert np.array_equal(np.array(th, np.float32), oth.astype(np.float32))


def _p(v):
    return ctypes.c_void_p(v)


# Fake, never dereferenced device addresses: validation must reject before any HIP call.
X, C, N, Q, S = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def test_encode_validation(L):
    e = L.tq_encode
    assert e(4, _p(X), 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_TYPE
    assert e(3, _p(X), 1, 1, 1, 100, _p(C), _p(N), 1, 0, None) == E_SHAPE
    assert e(3, _p(X), 1, 1, 1, 0, _p(C), _p(N), 1, 0, None) == E_SHAPE
    assert e(3, _p(X), -1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_SHAPE
    assert e(3, _p(X), 1, 1, 2, 128, _p(C), _p(N), 4, 3, None) == E_RANGE
    assert e(3, _p(X), 1, 1, 1, 128, _p(C), _p(N), 4, -1, None) == E_RANGE
    assert e(3, _p(X), 1, 1, 5, 128, _p(C), _p(N), 4, 0, None) == E_RANGE
    assert e(3, None, 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_NULL
    assert e(3, _p(X), 1, 1, 1, 128, None, _p(N), 1, 0, None) == E_NULL
    assert e(3, _p(X + 8), 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_ALIGN
    assert e(3, _p(X), 1, 1, 1, 128, _p(C + 4), _p(N), 1, 0, None) == E_ALIGN
    assert e(3, _p(X), 1, 1, 1, 128, _p(C), _p(N + 1), 1, 0, None) == E_ALIGN
    assert e(3, _p(X), 1, 1, 1, 128, _p(X + 128), _p(N), 1, 0, None) == E_ALIAS
    assert e(3, _p(X), 1, 1, 1, 128, _p(C), _p(C + 16), 1, 0, None) == E_ALIAS
    assert e(3, _p(X), 2, 3, 4, 256, _p(C), _p(X + 2 * 3 * 4 * 256 * 2 - 2), 9, 0, None) == E_ALIAS
    # zero work is a no-op success even with null pointers
    assert e(3, None, 0, 8, 16, 128, None, None, 16, 0, None) == OK
    assert e(2, None, 1, 1, 0, 128, None, None, 8, 8, None) == OK


def test_decode_validation(L):
    d = L.tq_decode
    assert d(1, _p(C), _p(N), 1, 1, 1, 128, 0, 1, _p(X), None) == E_TYPE
    assert d(3, _p(C), _p(N), 1, 1, 1, 129, 0, 1, _p(X), None) == E_SHAPE
    assert d(3, _p(C), _p(N), 1, 1, 4, 128, 2, 3, _p(X), None) == E_RANGE
    assert d(3, _p(C), None, 1, 1, 1, 128, 0, 1, _p(X), None) == E_NULL
    assert d(3, _p(C), _p(N), 1, 1, 1, 128, 0, 1, _p(X + 2), None) == E_ALIGN
    assert d(3, _p(C), _p(N), 1, 1, 1, 128, 0, 1, _p(C), None) == E_ALIAS
    assert d(3, None, None, 1, 1, 5, 128, 5, 0, None, None) == OK


def test_qk_validation(L):
    f = L.tq_qk_scores
    S4 = ctypes.cast(ctypes.c_void_p(S), ctypes.POINTER(ctypes.c_float))
    args = lambda **kw: dict(dict(t=3, c=_p(C), n=_p(N), B=1, Hkv=2, Tc=8, D=128, T=8, q=_p(Q),
                                  Hq=8, s=ctypes.c_float(1.0), o=S4), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["t"], a["c"], a["n"], a["B"], a["Hkv"], a["Tc"], a["D"], a["T"], a["q"],
                 a["Hq"], a["s"], a["o"], None)

    assert call(t=5) == E_TYPE
    assert call(Hq=7) == E_SHAPE
    assert call(Hkv=0) == E_SHAPE
    assert call(D=192) == E_SHAPE
    assert call(D=4096) == E_SHAPE
    assert call(T=9) == E_RANGE
    assert call(q=None) == E_NULL
    assert call(q=_p(Q + 2)) == E_ALIGN
    assert call(o=ctypes.cast(ctypes.c_void_p(S + 2), ctypes.POINTER(ctypes.c_float))) == E_ALIGN
    assert call(o=ctypes.cast(ctypes.c_void_p(Q), ctypes.POINTER(ctypes.c_float))) == E_ALIAS
    assert call(B=0, c=None, n=None, q=None) == OK
    assert call(T=0) == OK


def test_attn_workspace_bytes():
    """Depends on the sizes only; 4 + D floats (m, l, two spare, D values) per partial,
    one partial per row chunk of every (sequence, query head)."""
    ws = tq.tq_attn_workspace_bytes
    assert ws(3, 0, 8, 32768, 128, 32768, 32) == 0
    n16 = ws(3, 16, 8, 32768, 128, 32768, 32)
    assert n16 > 0 and n16 % (16 * 32 * 132 * 4) == 0
    n1 = ws(2, 1, 8, 32768, 128, 32768, 32)
    assert n1 > 0 and n1 % (32 * 132 * 4) == 0
    n256 = ws(2, 32, 4, 32768, 256, 32768, 16)
    assert n256 > 0 and n256 % (32 * 16 * 260 * 4) == 0
    for D in (384, 512, 100):
        with pytest.raises(tq.TQError):
            ws(3, 1, 8, 100, D, 100, 32)         # D not 128 or 256
    with pytest.raises(tq.TQError):
        ws(3, 1, 8, 100, 128, 0, 32)         # no rows
    with pytest.raises(tq.TQError):
        ws(3, 1, 8, 100, 128, 101, 32)       # T > Tc


def test_attn_workspace_chunking_limits():
    """The row chunking behind the workspace size: one 132-float record per (sequence,
    query head, chunk), at most 65535 chunks (the grid's y limit) however long the
    cache, and never more chunks than there are 256-row batches."""
    rec = 132 * 4
    tmax = 65535 * 1024   # longest attended range the library accepts
    for B, Hkv, G, T in [(1, 1, 1, 1), (1, 8, 4, 32768), (16, 8, 4, 32768), (3, 2, 12, 1000),
                         (1, 1, 1, tmax), (2, 4, 8, 33_000_000), (64, 8, 8, 131072)]:
        Hq = Hkv * G
        ws = tq.tq_attn_workspace_bytes(3, B, Hkv, T, 128, T, Hq)
        assert ws > 0 and ws % (B * Hq * rec) == 0, (B, Hkv, G, T)
        chunks = ws // (B * Hq * rec)
        assert 1 <= chunks <= 65535, (B, Hkv, G, T, chunks)
        assert chunks <= -(-T // 256), (B, Hkv, G, T, chunks)
        # a longer cache never needs fewer chunks
        if 2 * T <= tmax:
            assert tq.tq_attn_workspace_bytes(3, B, Hkv, 2 * T, 128, 2 * T, Hq) >= ws
    with pytest.raises(tq.TQError):
        tq.tq_attn_workspace_bytes(3, 1, 1, tmax + 1, 128, tmax + 1, 1)


def test_attn_validation(L):
    f = L.tq_attn_decode
    S4 = ctypes.cast(ctypes.c_void_p(S), ctypes.POINTER(ctypes.c_float))
    W = 0x60000000
    need = tq.tq_attn_workspace_bytes(3, 1, 2, 8, 128, 8, 8)
    args = lambda **kw: dict(dict(t=3, kc=_p(C), kn=_p(N), vc=_p(C + 0x1000000), vn=_p(N + 0x1000000),
                                  B=1, Hkv=2, Tc=8, D=128, T=8, q=_p(Q), Hq=8, s=ctypes.c_float(1.0),
                                  o=S4, w=_p(W), wb=need), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["t"], a["kc"], a["kn"], a["vc"], a["vn"], a["B"], a["Hkv"], a["Tc"], a["D"],
                 a["T"], a["q"], a["Hq"], a["s"], a["o"], a["w"], a["wb"], None)

    assert call(t=1) == E_TYPE
    assert call(Hq=7) == E_SHAPE
    assert call(D=384) == E_SHAPE
    assert call(D=256) == E_WORKSPACE      # valid sizes; the workspace is the head_dim-128 one
    assert call(T=0) == E_SHAPE
    assert call(T=9) == E_RANGE
    assert call(vc=None) == E_NULL
    assert call(w=None) == E_NULL
    assert call(vn=_p(N + 1)) == E_ALIGN
    assert call(w=_p(W + 8)) == E_ALIGN
    assert call(wb=need - 1) == E_WORKSPACE
    assert call(o=ctypes.cast(ctypes.c_void_p(C), ctypes.POINTER(ctypes.c_float))) == E_ALIAS
    assert call(w=_p(S)) == E_ALIAS
    assert call(B=0, kc=None, kn=None, vc=None, vn=None, q=None, w=None) == OK


def test_codebook_validation(L):
    buf = (ctypes.c_float * 8)()
    assert L.tq_codebook(4, buf, buf) == E_TYPE
    assert L.tq_codebook(3, None, buf) == E_NULL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 1, 4, 128), dtype=torch.float16)
    codes = torch.zeros((1, 1, 4, 1, 48), dtype=torch.uint8)
    norms = torch.zeros((1, 1, 4, 1), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        tq.tq_encode(3, x, codes, norms)


def test_rot_entry_points_validate_like_the_plain_ones(L):
    """The _rot calls take the plain call's arguments after the sign words and reject
    the same way before any HIP call; NULL signs are allowed (the plain rotation)."""
    W = (ctypes.c_uint32 * 4)(0xFFFFFFFF, 0, 1, 0x80000000)
    for signs in (W, None):
        e = L.tq_encode_rot
        assert e(4, signs, _p(X), 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_TYPE
        assert e(3, signs, _p(X), 1, 1, 1, 100, _p(C), _p(N), 1, 0, None) == E_SHAPE
        assert e(3, signs, _p(X), 1, 1, 2, 128, _p(C), _p(N), 4, 3, None) == E_RANGE
        assert e(3, signs, None, 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_NULL
        assert e(3, signs, _p(X + 8), 1, 1, 1, 128, _p(C), _p(N), 1, 0, None) == E_ALIGN
        assert e(3, signs, _p(X), 1, 1, 1, 128, _p(X + 128), _p(N), 1, 0, None) == E_ALIAS
        assert e(3, signs, None, 0, 8, 16, 128, None, None, 16, 0, None) == OK
        d = L.tq_decode_rot
        assert d(1, signs, _p(C), _p(N), 1, 1, 1, 128, 0, 1, _p(X), None) == E_TYPE
        assert d(3, signs, _p(C), _p(N), 1, 1, 4, 128, 2, 3, _p(X), None) == E_RANGE
        assert d(3, signs, _p(C), _p(N), 1, 1, 1, 128, 0, 1, _p(C), None) == E_ALIAS
        q = L.tq_qk_scores_rot
        S4 = ctypes.cast(ctypes.c_void_p(S), ctypes.POINTER(ctypes.c_float))
        assert q(3, signs, _p(C), _p(N), 1, 2, 8, 128, 8, _p(Q), 3, ctypes.c_float(1.0), S4, None) == E_SHAPE
        assert q(3, signs, _p(C), _p(N), 1, 2, 8, 128, 9, _p(Q), 4, ctypes.c_float(1.0), S4, None) == E_RANGE
        a = L.tq_attn_decode_rot
        assert a(3, signs, _p(C), _p(N), _p(C + 0x1000000), _p(N + 0x1000000), 1, 2, 8, 384, 8,
                 _p(Q), 4, ctypes.c_float(1.0), S4, _p(0x60000000), 1 << 20, None) == E_SHAPE
        assert a(3, signs, _p(C), _p(N), _p(C + 0x1000000), _p(N + 0x1000000), 1, 2, 8, 128, 8,
                 _p(Q), 4, ctypes.c_float(1.0), S4, _p(0x60000000), 0, None) == E_WORKSPACE


def test_sign_words_bit_layout():
    """Position p of a block <-> bit p % 32 of word p / 32; -1 (or True) sets the bit."""
    d = np.ones(128)
    d[[0, 31, 32, 100, 127]] = -1
    w = list(tq.sign_words(d))
    assert w == [0x80000001, 0x00000001, 0x00000000, 0x80000010]
    assert list(tq.sign_words([v < 0 for v in d])) == w
    assert list(tq.sign_words(np.ones(128))) == [0, 0, 0, 0]
    with pytest.raises(ValueError):
        tq.sign_words(np.ones(127))
    with pytest.raises(ValueError):
        tq.sign_words(np.full(128, 0.5))
    # words from an earlier call pass through as they are (no conversion per launch)
    words = tq.sign_words(d)
    assert tq.sign_words(words) is words
    with pytest.raises(ValueError):
        tq.sign_words((ctypes.c_uint32 * 3)(1, 2, 3))


def test_record_validation(L):
    p, u = L.tq_pack_records, L.tq_unpack_records
    R = 0x70000000
    assert p(4, _p(C), _p(N), 8, _p(R), None) == E_TYPE
    assert p(3, _p(C), _p(N), -1, _p(R), None) == E_SHAPE
    assert p(3, _p(C), _p(N), 1 << 31, _p(R), None) == E_SHAPE
    assert p(3, None, _p(N), 8, _p(R), None) == E_NULL
    assert p(3, _p(C + 8), _p(N), 8, _p(R), None) == E_ALIGN
    assert p(3, _p(C), _p(N + 1), 8, _p(R), None) == E_ALIGN
    assert p(3, _p(C), _p(N), 8, _p(R + 2), None) == E_ALIGN
    assert p(3, _p(C), _p(N), 8, _p(C + 16), None) == E_ALIAS
    assert p(2, None, None, 0, None, None) == OK
    assert u(1, _p(R), 8, _p(C), _p(N), None) == E_TYPE
    assert u(3, _p(R), -5, _p(C), _p(N), None) == E_SHAPE
    assert u(3, _p(R), 8, _p(C), None, None) == E_NULL
    assert u(3, _p(R + 4), 8, _p(C), _p(N), None) == E_ALIGN
    assert u(3, _p(R), 8, _p(C), _p(C + 384 - 2), None) == E_ALIAS      # norms inside the codes
    assert u(3, _p(R), 8, _p(R + 16), _p(N), None) == E_ALIAS
    assert u(3, None, 0, None, None, None) == OK


def test_timing_hook_sets_and_clears_without_a_gpu(L):
    """tq_time_next_launch only stores per-thread state: arming and clearing it needs
    no device, and the binding refuses a torch event that has no HIP event yet."""
    import torch
    assert L.tq_time_next_launch(ctypes.c_void_p(0x1000), None) == OK
    assert L.tq_time_next_launch(None, None) == OK     # cleared: no launch will touch 0x1000
    with pytest.raises(ValueError, match="record it once"):
        tq.tq_time_next_launch(torch.cuda.Event(enable_timing=True), None)
    tq.tq_time_next_launch(None, None)


def test_launch_failure_returns_err_device(L):
    """A call that passes validation reaches the launch, and a launch that HIP reports
    as failed returns TQ_ERR_DEVICE.  Forced on a host without a GPU, where every launch
    fails (the pointers are never dereferenced); skipped wherever a GPU is visible."""
    import torch
    if torch.cuda.device_count() > 0 or os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is visible: a launch would run")
    E_DEVICE = -7
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    for bits in (3, 2):
        assert L.tq_encode(bits, _p(X), 1, 2, 16, 128, _p(C), _p(N), 16, 0, None) == E_DEVICE
        assert L.tq_decode(bits, _p(C), _p(N), 1, 2, 16, 128, 0, 16, _p(X), None) == E_DEVICE
        assert L.tq_qk_scores(bits, _p(C), _p(N), 1, 2, 16, 128, 16, _p(Q), 8, ctypes.c_float(0.1),
                              _p(S), None) == E_DEVICE
        ws = L.tq_attn_workspace_bytes(bits, 1, 2, 16, 128, 16, 8)
        assert ws > 0
        assert L.tq_attn_decode(bits, _p(C), _p(N), _p(C + 0x1000000), _p(N + 0x1000000), 1, 2, 16,
                                128, 16, _p(Q), 8, ctypes.c_float(0.1), _p(S), _p(0x60000000), ws,
                                None) == E_DEVICE
        assert L.tq_pack_records(bits, _p(C), _p(N), 64, _p(0x60000000), None) == E_DEVICE
        assert L.tq_unpack_records(bits, _p(0x60000000), 64, _p(C), _p(N), None) == E_DEVICE
    assert tq.tq_status_string(E_DEVICE).startswith("TQ_ERR_DEVICE")


def test_attn_noalloc_validation(L):
    """tq_attn_decode_noalloc checks its arguments like tq_attn_decode, and refuses sizes
    whose partials would not fit the static scratch array (TQ_ERR_WORKSPACE), all before
    any HIP call."""
    f = L.tq_attn_decode_noalloc
    sc = ctypes.c_float(0.1)
    K2, N2 = C + 0x1000000, N + 0x1000000
    assert f(4, None, _p(C), _p(N), _p(K2), _p(N2), 1, 2, 16, 128, 16, _p(Q), 8, sc, _p(S), None) == E_TYPE
    assert f(3, None, _p(C), _p(N), _p(K2), _p(N2), 1, 2, 16, 384, 16, _p(Q), 8, sc, _p(S), None) == E_SHAPE
    assert f(3, None, _p(C), _p(N), _p(K2), _p(N2), 1, 2, 16, 128, 17, _p(Q), 8, sc, _p(S), None) == E_RANGE
    assert f(3, None, None, _p(N), _p(K2), _p(N2), 1, 2, 16, 128, 16, _p(Q), 8, sc, _p(S), None) == E_NULL
    assert f(3, None, _p(C + 8), _p(N), _p(K2), _p(N2), 1, 2, 16, 128, 16, _p(Q), 8, sc, _p(S), None) == E_ALIGN
    assert f(3, None, _p(C), _p(N), _p(K2), _p(N2), 1, 2, 16, 128, 16, _p(Q), 8, sc, _p(C), None) == E_ALIAS
    assert f(3, None, None, None, None, None, 0, 2, 16, 128, 16, None, 8, sc, None, None) == OK
    # 512 sequences x 32 heads of 256 rows: 8.65 MB of partials, beyond the 8 MiB array
    assert L.tq_attn_workspace_bytes(3, 512, 8, 256, 128, 256, 32) > tq.TQ_ATTN_SCRATCH_BYTES
    assert f(3, None, _p(C), _p(N), _p(K2), _p(N2), 512, 8, 256, 128, 256, _p(Q), 32, sc, _p(S),
             None) == E_WORKSPACE
    import re
    m = re.search(r"#define TQ_ATTN_SCRATCH_BYTES \((\d+) << (\d+)\)", open(tq.HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == tq.TQ_ATTN_SCRATCH_BYTES
