"""Pins for the oracle's FP8-E4M3 decoding and FP8-pool attention."""

import math

import numpy as np
import torch

import oracle
import workloads


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_fp8_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_decode_hand_values():
    d = lambda c: float(oracle.decode_fp8_e4m3(np.array([c], np.uint8))[0])
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x38) == 1.0 and d(0xB8) == -1.0            # e = 7, m = 0
    assert d(0x3F) == 1.875                              # e = 7, m = 7
    assert d(0x7E) == 448.0                              # largest finite
    assert d(0x01) == 2.0 ** -9                          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9                      # largest subnormal
    assert d(0x08) == 2.0 ** -6                          # smallest normal
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))


def test_fp8_attention_is_attention_of_the_dequantised_pools():
    w = workloads.build(3, 10, 2, 32, [1, 130, 257], seed=5, max_pages=3, pool="packed")
    f = workloads.quantize_fp8(w)
    k = oracle.decode_fp8_e4m3(f.k_codes.numpy()) * float(np.float32(f.k_scale))
    v = oracle.decode_fp8_e4m3(f.v_codes.numpy()) * float(np.float32(f.v_scale))
    a = oracle.paged_decode_attention_fp8(w.q, f.k_codes, f.v_codes, f.k_scale, f.v_scale,
                                          w.block_table, w.context_lens, w.scale)
    b = oracle.paged_decode_attention(w.q, k, v, w.block_table, w.context_lens, w.scale)
    assert np.array_equal(a, b)
    # quantisation error stays small against the BF16 original
    c = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert np.max(np.abs(a - c)) < 0.2


def test_v_scale_is_linear_and_ctx1_returns_the_scaled_row():
    w = workloads.build(2, 8, 1, 16, [1, 9], seed=6, max_pages=1, pool="packed")
    f = workloads.quantize_fp8(w)
    o1 = oracle.paged_decode_attention_fp8(w.q, f.k_codes, f.v_codes, f.k_scale, 1.0,
                                           w.block_table, w.context_lens, w.scale)
    o2 = oracle.paged_decode_attention_fp8(w.q, f.k_codes, f.v_codes, f.k_scale, 0.5,
                                           w.block_table, w.context_lens, w.scale)
    assert np.array_equal(o2, 0.5 * o1)    # a power-of-two scale is exact
    page = int(w.block_table[0, 0])
    row = oracle.decode_fp8_e4m3(f.v_codes[page, 0, 0].numpy())
    for hq in range(8):
        assert np.array_equal(o1[0, hq], row)


def test_quantisation_recipe():
    w = workloads.build(2, 8, 2, 16, [40, 100], seed=8, max_pages=1, pool="packed")
    f = workloads.quantize_fp8(w)
    assert f.k_codes.dtype == torch.uint8 and f.k_codes.shape == w.k_cache.shape
    vals = oracle.decode_fp8_e4m3(f.k_codes.numpy())
    assert np.nanmax(np.abs(vals)) == 448.0           # the largest |x| maps to the top code
    rel = np.abs(vals * f.k_scale - w.k_cache.float().numpy())
    assert np.max(rel) <= 2.0 ** -4 * np.max(np.abs(w.k_cache.float().numpy())) + 1e-6
