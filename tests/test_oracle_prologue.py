"""Pins for the oracle's attention prologue (QK-norm, NeoX RoPE, KV write)."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(7)


def test_rms_norm_matches_torch_rms_norm():
    # the library routine, in FP64, per head over the last axis
    x = RNG.standard_normal((5, 3, 128))
    w = RNG.standard_normal(128)
    for eps in (1e-6, 1e-2):
        ref = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(w), eps=eps).numpy()
        got = oracle.rms_norm_heads(x, w, np.float32(eps))
        assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))  # eps widened from FP32


def test_rms_norm_closed_forms():
    w = RNG.standard_normal(64)
    c, eps = 3.0, 1e-6
    y = oracle.rms_norm_heads(np.full((1, 64), c), w, eps)
    assert np.allclose(y[0], c / math.sqrt(c * c + float(np.float32(eps))) * w, rtol=1e-15, atol=0)
    x = RNG.standard_normal((2, 64))
    # scale invariance when eps is negligible
    assert np.allclose(oracle.rms_norm_heads(1e3 * x, w, 0.0), oracle.rms_norm_heads(x, w, 0.0),
                       rtol=1e-12, atol=0)
    # unit weights give mean(y^2) = 1 (eps = 0)
    y = oracle.rms_norm_heads(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)


def test_rope_worked_example_pairs_halves_and_rotates_forward():
    # D = 4, x = e_0, position 1, base 100: theta_0 = 1 rad, theta_1 = 100^(-1/2) = 0.1.
    # NeoX pairs dim 0 with dim 2 (the halves), rotating by +theta:
    # out = [cos 1, 0, sin 1, 0]; adjacent-pair (interleaved) RoPE would give
    # [cos 1, sin 1, 0, 0].
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    out = oracle.rope_neox(x, [1], 100.0, 1.0)[0, 0]
    assert np.allclose(out, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], rtol=0, atol=1e-15)
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    out = oracle.rope_neox(x, [1], 100.0, 1.0)[0, 0]
    assert np.allclose(out, [0.0, math.cos(0.1), 0.0, math.sin(0.1)], rtol=0, atol=1e-15)
    # the frequency scale divides the angle: scale 2 at position 2 equals position 1
    a = oracle.rope_neox(np.array([[[0.3, -1.2, 0.7, 2.0]]]), [2], 100.0, 2.0)
    b = oracle.rope_neox(np.array([[[0.3, -1.2, 0.7, 2.0]]]), [1], 100.0, 1.0)
    assert np.allclose(a, b, rtol=0, atol=1e-15)


def test_rope_angles_closed_form():
    th = oracle.rope_angles([0, 1, 4095], 128, 1e6, 1.0)
    assert th.shape == (3, 64)
    assert np.all(th[0] == 0)
    assert th[1, 0] == 1.0
    assert math.isclose(th[1, 1], 10.0 ** (-6 * 2 / 128), rel_tol=1e-15)
    assert math.isclose(th[2, 63], 4095 * 10.0 ** (-6 * 126 / 128), rel_tol=1e-14)


def test_rope_properties():
    x = RNG.standard_normal((4, 3, 128))
    y = RNG.standard_normal((4, 3, 128))
    base = 1e6
    # position 0 is the identity
    assert np.array_equal(oracle.rope_neox(x, [0] * 4, base, 1.0), x)
    # each (i, i + D/2) pair keeps its length
    r = oracle.rope_neox(x, [3, 70, 1000, 4095], base, 1.0)
    assert np.allclose(r[..., :64] ** 2 + r[..., 64:] ** 2, x[..., :64] ** 2 + x[..., 64:] ** 2,
                       rtol=1e-12)
    # composition: rotating by a then b is rotating by a + b
    rab = oracle.rope_neox(oracle.rope_neox(x, [5, 6, 7, 8], base, 1.0), [10, 20, 30, 40], base, 1.0)
    assert np.allclose(rab, oracle.rope_neox(x, [15, 26, 37, 48], base, 1.0), atol=1e-12)
    # relative position: q.k depends only on the position difference
    d1 = np.sum(oracle.rope_neox(x, [100] * 4, base, 1.0) * oracle.rope_neox(y, [40] * 4, base, 1.0), -1)
    d2 = np.sum(oracle.rope_neox(x, [1100] * 4, base, 1.0) * oracle.rope_neox(y, [1040] * 4, base, 1.0), -1)
    assert np.allclose(d1, d2, atol=1e-10)


def test_prologue_writes_normed_rotated_k_and_raw_v():
    T, Hq, Hkv, D, N, P = 5, 6, 2, 128, 3, 128
    q = RNG.standard_normal((T, Hq, D))
    k = RNG.standard_normal((T, Hkv, D))
    v = RNG.standard_normal((T, Hkv, D))
    wq, wk = RNG.standard_normal(D), RNG.standard_normal(D)
    kc = RNG.standard_normal((N, P, Hkv, D))
    vc = RNG.standard_normal((N, P, Hkv, D))
    pos = [7, 8, 9, 300, 4095]
    slots = [7, 8, -1, 2 * P + 5, P]
    qo, kc2, vc2 = oracle.attention_prologue(q, k, v, wq, wk, pos, slots, 1e-6, 1e6, 1.0, kc, vc)
    assert np.allclose(qo, oracle.rope_neox(oracle.rms_norm_heads(q, wq, 1e-6), pos, 1e6, 1.0))
    kr = oracle.rope_neox(oracle.rms_norm_heads(k, wk, 1e-6), pos, 1e6, 1.0)
    touched = np.zeros((N, P), bool)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        page, off = divmod(sl, P)
        touched[page, off] = True
        assert np.array_equal(kc2[page, off], kr[t])
        assert np.array_equal(vc2[page, off], v[t])      # V goes in untouched
    assert np.array_equal(kc2[~touched], kc[~touched])
    assert np.array_equal(vc2[~touched], vc[~touched])


def test_round_bf16_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-140, 120, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()   # one rounding from FP32
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)
    got = oracle.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8),
                                      1 + 2.0 ** -8 + 2.0 ** -40, 0.0]))
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7, 0.0]


def test_fp8_prologue_writes_codes_of_the_bf16_rows():
    T, Hq, Hkv, D, N, P = 6, 4, 2, 128, 3, 128
    rng = np.random.default_rng(42)
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = torch.from_numpy(rng.standard_normal((T, Hkv, D))).to(torch.bfloat16)
    wq, wk = rng.standard_normal(D), rng.standard_normal(D)
    kc = rng.integers(0, 256, (N, P, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (N, P, Hkv, D), dtype=np.uint8)
    pos = [7, 8, 9, 300, 4095, 12]
    slots = [7, 8, -1, 2 * P + 5, P, N * P]
    ks, vs = 0.05, 0.02          # |K| / ks and |v| / vs stay below 448 (no saturation)
    qo, kc2, vc2 = oracle.attention_prologue_fp8(q, k, v, wq, wk, pos, slots, 1e-6, 1e6, 1.0,
                                                 ks, vs, kc, vc)
    qb, _, _ = oracle.attention_prologue(q, k, v, wq, wk, pos, slots, 1e-6, 1e6, 1.0,
                                         np.zeros((N, P, Hkv, D)), np.zeros((N, P, Hkv, D)))
    assert np.array_equal(qo, qb)
    kr = oracle.rope_neox(oracle.rms_norm_heads(k, wk, 1e-6), pos, 1e6, 1.0)
    touched = np.zeros((N, P), bool)
    for t, sl in enumerate(slots):
        if not 0 <= sl < N * P:
            continue
        page, off = divmod(sl, P)
        touched[page, off] = True
        # V: torch's own FP8 cast of the FP32 quotient (an independent rounding)
        vq = (v[t].float() / torch.tensor(vs, dtype=torch.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(vc2[page, off], vq.view(torch.uint8).numpy())
        # K: within half an E4M3 step of the exact rotated row, plus BF16 rounding
        dec = oracle.decode_fp8_e4m3(kc2[page, off]) * float(np.float32(ks))
        err = np.abs(dec - kr[t])
        assert np.all(err <= (2.0 ** -4 + 2.0 ** -8) * np.abs(kr[t]) * 1.001 + 2.0 ** -10 * ks)
    assert np.array_equal(kc2[~touched], kc[~touched])
    assert np.array_equal(vc2[~touched], vc[~touched])


def test_planted_mistakes_fail_the_pins():
    # adjacent-pair (GPT-J) rotation and a backwards rotation both miss the
    # worked example; a norm that forgets the weight misses torch's rms_norm
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    want = np.array([math.cos(1.0), 0.0, math.sin(1.0), 0.0])
    th = 1.0
    interleaved = np.array([math.cos(th), math.sin(th), 0.0, 0.0])
    backwards = np.array([math.cos(th), 0.0, -math.sin(th), 0.0])
    assert not np.allclose(interleaved, want) and not np.allclose(backwards, want)
    assert np.allclose(oracle.rope_neox(x, [1], 100.0, 1.0)[0, 0], want)
    xx = RNG.standard_normal((2, 16))
    w = RNG.standard_normal(16)
    no_weight = xx / np.sqrt(np.mean(xx * xx, -1, keepdims=True) + 1e-6)
    ref = F.rms_norm(torch.from_numpy(xx), (16,), weight=torch.from_numpy(w), eps=1e-6).numpy()
    assert not np.allclose(no_weight, ref, atol=1e-3)
