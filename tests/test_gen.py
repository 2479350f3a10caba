"""The seeded input generator shared by the oracle side and the GPU side (CPU only).

Both sides of every parity test draw their inputs here, so these tests pin what the
generator promises: splitmix64 as published, a counter-based stream (value (h, t, d) of
layer l is counter ((l H + h) T_total + t_offset + t) D + d, so any slice regenerates
the same values as the whole tensor), the workloads' outlier channels and row scales,
and bit-for-bit determinism.
"""
import numpy as np
import pytest
import torch

import gen

# splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
# OOPSLA 2014; the reference C code of the generator): outputs for seed 1234567, the
# values every implementation of the published constants produces.
M64 = (1 << 64) - 1


def splitmix64_mix(x):
    """One splitmix64 output from state x (the state advanced by the golden gamma, then
    the two xor-shift-multiply rounds and a final xor-shift), in Python integers."""
    z = (x + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_matches_the_published_sequence():
    """The generator's sequence form, state s_k = seed + k * gamma, gives the published
    outputs for seed 1234567; the library's scalar hash is its first step."""
    seq, s = [], 1234567
    for _ in range(5):
        seq.append(splitmix64_mix(s))
        s = (s + 0x9E3779B97F4A7C15) & M64
    assert seq == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]
    assert gen._splitmix64_int(1234567) == seq[0]
    assert int(gen.bits64(1234567, 1).numpy().astype(np.uint64)[0]) == seq[0]


@pytest.mark.parametrize("key", [0, 1234567, (1 << 63) + 12345, M64 - 3, 0x0123456789ABCDEF])
def test_counter_hash_in_int64_tensors_matches_python_integers(key):
    """bits64 computes splitmix64 of (key + counter) in int64 tensor arithmetic (wrapping
    adds and products, logical shifts emulated on signed words): it must equal the same
    function in unbounded Python integers, across the sign bit and the 2^64 wrap."""
    off = 2 ** 40 - 3
    got = gen.bits64(key, 64, off).numpy().astype(np.uint64)
    ref = np.array([splitmix64_mix((key + off + k) & M64) for k in range(64)], dtype=np.uint64)
    np.testing.assert_array_equal(got, ref)


def test_uniform_and_normal_are_functions_of_the_counter():
    key = gen.stream_key(5, 1, 2)
    u = gen.uniform(key, 1000, 77)
    assert float(u.min()) >= 0.0 and float(u.max()) < 1.0
    # a window of counters regenerates the same values
    assert torch.equal(gen.uniform(key, 100, 500), u[423:523])
    n = gen.normal(key, 1000, 77)
    assert torch.equal(gen.normal(key, 10, 1000), n[923:933])
    # Box-Muller by hand from the same 64-bit counter hash
    z = gen.bits64(key, 1000, 77).numpy().astype(np.uint64)
    u1 = ((z >> np.uint64(32)).astype(np.float64) + 0.5) / 4294967296.0
    u2 = (z & np.uint64(0xFFFFFFFF)).astype(np.float64) / 4294967296.0
    ref = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    # (torch's and numpy's log / cos may differ in the last bit)
    np.testing.assert_allclose(n.numpy(), ref, rtol=1e-13, atol=1e-13)


def test_normal_statistics():
    n = gen.normal(gen.stream_key(9, 0), 200000).numpy()
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1.0) < 0.01


@pytest.mark.parametrize("spec", [gen.KVSpec(), gen.KVSpec(n_outliers=3, row_scale=True),
                                  gen.KVSpec(n_outliers=5, student_t3=True)])
def test_slices_regenerate_the_whole(spec):
    """Rows [t0, t0 + T) of a tensor of T_total rows, drawn alone, equal the same rows of
    the whole: the decode-step append and the per-layer streaming of the full-size
    checks rely on this."""
    whole = gen.kv_layer(3, "K", spec, 2, 4, 40, 256)
    for t0, T in ((0, 40), (5, 1), (39, 1), (17, 9)):
        part = gen.kv_layer(3, "K", spec, 2, 4, T, 256, t_offset=t0, T_total=40)
        assert torch.equal(part.view(torch.int16), whole[:, t0:t0 + T].view(torch.int16))


def test_plain_layer_is_the_counter_stream():
    """Without outliers or row scales, value (h, t, d) of layer l is normal() at counter
    ((l H + h) T + t) D + d of the tensor's element stream, rounded to fp16."""
    l, H, T, D = 3, 2, 5, 128
    x = gen.kv_layer(11, "V", gen.KVSpec(), l, H, T, D)
    key = gen.stream_key(11, gen.TENSOR_IDS["V"], 0)
    ref = gen.normal(key, H * T * D, l * H * T * D).view(H, T, D).to(torch.float16)
    assert torch.equal(x.view(torch.int16), ref.view(torch.int16))


def test_outlier_channels_and_row_scale():
    """The chosen channels of a (layer, head) carry gain x the plain stream; the others
    are the plain stream times the row scale 0.5 * 8^u in [0.5, 4)."""
    spec = gen.KVSpec(n_outliers=3, row_scale=True)
    l, H, T, D = 1, 3, 64, 128
    x = gen.kv_layer(4, "K", spec, l, H, T, D).double()
    plain = gen.kv_layer(4, "K", gen.KVSpec(), l, H, T, D).double()
    key = gen.stream_key(4, gen.TENSOR_IDS["K"], 2)
    for h in range(H):
        ch = gen.outlier_channels(4, "K", l, h, D, 3)
        assert len(set(ch.tolist())) == 3
        u = gen.uniform(key, T, (l * H + h) * T)
        s = 0.5 * torch.pow(8.0, u)
        assert float(s.min()) >= 0.5 and float(s.max()) < 4.0
        other = [c for c in range(D) if c not in set(ch.tolist())]
        # fp16 rounding of both sides: compare within the fp16 spacing
        np.testing.assert_allclose(x[h][:, other].numpy(), (plain[h][:, other] * s[:, None]).numpy(),
                                   rtol=2e-3, atol=1e-6)
        np.testing.assert_allclose(x[h][:, ch].numpy(), (plain[h][:, ch] * 20.0 * s[:, None]).numpy(),
                                   rtol=2e-3, atol=1e-6)


def test_deterministic():
    for name in ("one_layer", "head_dim_256"):
        w = gen.WORKLOADS[name]
        a = gen.kv_layer(w.seed, "K", w.spec, 0, w.H, 64, w.D, T_total=w.T)
        b = gen.kv_layer(w.seed, "K", w.spec, 0, w.H, 64, w.D, T_total=w.T)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
