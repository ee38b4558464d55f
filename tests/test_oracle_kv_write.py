"""Pins for the oracle's paged KV write (the slot-mapping scatter)."""

import numpy as np
import torch

import oracle
import workloads


def _flat_write_reference(cache, new, slots):
    # the pool as one flat array of [Hkv*D] rows: row index = slot
    N, P, H, D = cache.shape
    flat = cache.reshape(N * P * H * D).copy()
    for t, s in enumerate(slots):
        if 0 <= s < N * P:
            flat[s * H * D:(s + 1) * H * D] = new[t].reshape(H * D)
    return flat.reshape(N, P, H, D)


def test_write_matches_flat_row_addressing():
    rng = np.random.default_rng(3)
    N, P, H, D, T = 6, 4, 2, 8, 9
    k = rng.standard_normal((N, P, H, D))
    v = rng.standard_normal((N, P, H, D))
    kn = rng.standard_normal((T, H, D))
    vn = rng.standard_normal((T, H, D))
    slots = np.array([0, 23, 5, -1, 7, 4 * 6, 11, -5, 12])   # includes padding and one past the pool
    k2, v2 = oracle.paged_kv_write(k, v, kn, vn, slots)
    assert np.array_equal(k2, _flat_write_reference(k, kn, slots))
    assert np.array_equal(v2, _flat_write_reference(v, vn, slots))
    # inputs untouched; rows no valid slot names unchanged
    assert not np.shares_memory(k2, k)
    written = {int(s) for s in slots if 0 <= s < N * P}
    for s in range(N * P):
        if s not in written:
            assert np.array_equal(k2[s // P, s % P], k[s // P, s % P])


def test_write_then_attend_sees_the_new_token():
    # decode step: write token ctx-1 of every sequence, then attend over ctx
    w = workloads.build(3, 10, 2, 16, [5, 129, 1], seed=9, max_pages=2, pool="packed")
    ctx = w.context_lens.numpy()
    slots = np.array([int(w.block_table[b, (c - 1) // 128]) * 128 + (c - 1) % 128
                      for b, c in enumerate(ctx)])
    gen = torch.Generator().manual_seed(1)
    kn = torch.randn(3, 2, 16, generator=gen).to(torch.bfloat16)
    vn = torch.randn(3, 2, 16, generator=gen).to(torch.bfloat16)
    k2, v2 = oracle.paged_kv_write(w.k_cache.float().numpy(), w.v_cache.float().numpy(),
                                   kn.float().numpy(), vn.float().numpy(), slots)
    out = oracle.paged_decode_attention(w.q, k2, v2, w.block_table, w.context_lens, w.scale)
    # sequence 2 has ctx 1: its output is exactly the V row just written
    for hq in range(10):
        assert np.array_equal(out[2, hq], vn.float().numpy()[2, hq // 5].astype(np.float64))
