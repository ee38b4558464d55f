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


# ---- encoding (the FP8 KV write) ---------------------------------------------

def _enc(*vals):
    return oracle.encode_fp8_e4m3(np.array(vals, dtype=np.float32)).tolist()


def test_encode_round_trips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_fp8_e4m3(codes)
    finite = ~np.isnan(vals)
    back = oracle.encode_fp8_e4m3(vals[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])          # -0.0 included: 0x80


def test_encode_hand_values():
    # ties between neighbours go to the even code (even mantissa)
    assert _enc(1.0625, 1.1875, -1.0625) == [0x38, 0x3A, 0xB8]
    assert _enc(1.0625 + 2.0 ** -20, 1.1875 - 2.0 ** -20) == [0x39, 0x39]
    # subnormals: 2^-10 is the midpoint of 0 and 2^-9, 3*2^-10 of codes 1 and 2
    assert _enc(2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -10 + 2.0 ** -30) == [0x00, 0x02, 0x01]
    assert _enc(1e-40, -1e-40, -0.0, 0.0) == [0x00, 0x80, 0x80, 0x00]
    # saturation: no infinity in the format, everything past 448 stays 448
    assert _enc(448.0, 460.0, 464.0, 1e30, np.inf, -np.inf) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert _enc(np.nan) == [0x7F]
    assert _enc(240.0, 15.0) == [0x77, 0x57]            # 1.875*2^7 and 1.875*2^3


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(21)
    y = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1.0, 30.0, 300.0)])
    y = y.astype(np.float32)
    codes = oracle.encode_fp8_e4m3(y)
    table = oracle.decode_fp8_e4m3(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(table)
    cand = np.nonzero(ok)[0]
    dist = np.abs(table[cand][None, :] - y.astype(np.float64)[:, None])
    best = dist.min(axis=1)
    mine = np.abs(oracle.decode_fp8_e4m3(codes) - y.astype(np.float64))
    assert np.array_equal(mine, np.minimum(best, np.inf))
    assert np.array_equal(np.signbit(oracle.decode_fp8_e4m3(codes)) | (codes == 0),
                          np.signbit(y) | (codes == 0))


def test_encode_matches_torch_conversion_inside_the_range():
    # torch's float8_e4m3fn cast rounds to nearest even; it differs from the
    # saturating encoder only past 464, where it gives NaN
    rng = np.random.default_rng(22)
    v = oracle.decode_fp8_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    y = np.concatenate([mids, -mids, rng.uniform(-448, 448, 20000).astype(np.float32),
                        (rng.standard_normal(20000) * 0.01).astype(np.float32)])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8_e4m3(y), ref)


def test_quantize_takes_the_quotient_in_fp32():
    # a power-of-two scale divides exactly
    x = np.array([1.5, -3.0, 100.0, 0.007], np.float32)
    assert np.array_equal(oracle.quantize_fp8_e4m3(x, 0.5), oracle.encode_fp8_e4m3(2 * x))
    # cases where the FP32 quotient lands exactly on a midpoint that the exact
    # quotient misses: the code is the tie's even neighbour, not the exact
    # quotient's nearest value
    rng = np.random.default_rng(23)
    v = oracle.decode_fp8_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (v[1:] + v[:-1]) / 2
    found = 0
    for _ in range(20000):
        m = mids[rng.integers(8, len(mids))]
        s = np.float32(rng.uniform(0.5, 2.0))
        x = np.float32(m * float(s))
        if float(x / s) != m or float(x) == m * float(s):
            continue
        code = int(oracle.quantize_fp8_e4m3(np.array([x]), s)[0])
        tie = int(oracle.encode_fp8_e4m3(np.array([m], np.float32))[0])
        assert code == tie and code % 2 == 0
        lo = int(np.searchsorted(v, m)) - 1            # codes lo, lo + 1 enclose m
        exact = lo + 1 if float(x) > m * float(s) else lo   # FP64 compare is exact here
        found += exact != tie
    assert found > 20


def test_kv_write_fp8_is_the_write_of_the_codes():
    rng = np.random.default_rng(24)
    N, P, H, D, T = 5, 128, 2, 16, 7
    kc = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    kn = torch.from_numpy(rng.standard_normal((T, H, D)) * 3).to(torch.bfloat16)  # |x|/s < 448
    vn = torch.from_numpy(rng.standard_normal((T, H, D))).to(torch.bfloat16)
    slots = np.array([0, 639, 5, -1, 128 * 5, 300, 77])
    k2, v2 = oracle.paged_kv_write_fp8(kc, vc, kn, vn, 0.05, 0.5, slots)
    # reference: torch's own conversion of the FP32 quotient (all in range)
    kq = (kn.float() / torch.tensor(0.05, dtype=torch.float32)).to(torch.float8_e4m3fn)
    vq = (vn.float() / 0.5).to(torch.float8_e4m3fn)
    for t, s in enumerate(slots):
        if 0 <= s < N * P:
            assert np.array_equal(k2[s // P, s % P], kq[t].view(torch.uint8).numpy())
            assert np.array_equal(v2[s // P, s % P], vq[t].view(torch.uint8).numpy())
    untouched = np.ones(N * P, bool)
    untouched[[s for s in slots if 0 <= s < N * P]] = False
    assert np.array_equal(k2.reshape(N * P, H, D)[untouched], kc.reshape(N * P, H, D)[untouched])
    assert np.array_equal(v2.reshape(N * P, H, D)[untouched], vc.reshape(N * P, H, D)[untouched])
    # decoded values are within half a step of the originals (relative 2^-4)
    dec = oracle.decode_fp8_e4m3(k2[0, 0]) * float(np.float32(0.05))
    x = kn[0].double().numpy()
    assert np.all(np.abs(dec - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * 0.05)
