"""GPU parity of the paged KV write (bit-exact against the oracle's index write)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import announce, assert_parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from paged_gqa_attention_amd import pagedattn  # noqa: F401


def _bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("Hkv,D,T", [(8, 128, 16), (8, 128, 3000), (2, 256, 257), (1, 8, 5), (3, 64, 40)])
def test_write_bit_exact(Hkv, D, T):
    announce(f"kv write Hkv={Hkv} D={D} T={T}")
    from paged_gqa_attention_amd import pagedattn as pa
    N, P = 40, 128
    gen = torch.Generator().manual_seed(T + D)
    k = torch.randn(N, P, Hkv, D, generator=gen).to(torch.bfloat16)
    v = torch.randn(N, P, Hkv, D, generator=gen).to(torch.bfloat16)
    kn = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
    # distinct slots, some padding (-1, -7) and some past the pool
    slots = torch.randperm(N * P, generator=gen)[:T].to(torch.int32)
    slots[::7] = -1
    slots[3::11] = N * P + 5
    if T > 2:
        slots[1] = -7
    kd, vd = k.cuda(), v.cuda()
    pa.pa_kv_write(kn.cuda(), vn.cuda(), slots.cuda(), kd, vd)
    torch.cuda.synchronize()
    rk, rv = oracle.paged_kv_write(_bf16_bits(k), _bf16_bits(v), _bf16_bits(kn), _bf16_bits(vn),
                                   slots.numpy())
    assert np.array_equal(_bf16_bits(kd), rk)
    assert np.array_equal(_bf16_bits(vd), rv)


def test_empty_write_is_a_no_op():
    from paged_gqa_attention_amd import pagedattn as pa
    k = torch.randn(2, 128, 8, 128, device="cuda").to(torch.bfloat16)
    v = k.clone()
    before = k.clone()
    e = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    pa.pa_kv_write(e, e, torch.empty(0, dtype=torch.int32, device="cuda"), k, v)
    torch.cuda.synchronize()
    assert torch.equal(k, before)


def test_decode_step_write_then_attend():
    # one decode step: write every sequence's new token at position ctx-1,
    # then attend over ctx tokens; compare with the oracle doing the same
    announce("decode step: write + attend")
    from paged_gqa_attention_amd import pagedattn as pa
    w = workloads.config(2)
    B, Hkv, D = 16, 8, 128
    gen = torch.Generator().manual_seed(77)
    kn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    ctx = w.context_lens
    slots = torch.tensor([int(w.block_table[b, (int(c) - 1) // 128]) * 128 + (int(c) - 1) % 128
                          for b, c in enumerate(ctx)], dtype=torch.int32)
    dev = "cuda:0"
    kd, vd = w.k_cache.to(dev), w.v_cache.to(dev)
    pa.pa_kv_write(kn.to(dev), vn.to(dev), slots.to(dev), kd, vd)
    out = pa.pa_decode(w.q.to(dev), kd, vd, w.block_table.to(dev), ctx.to(dev), scale=w.scale)
    torch.cuda.synchronize()
    k2, v2 = oracle.paged_kv_write(w.k_cache.float().numpy(), w.v_cache.float().numpy(),
                                   kn.float().numpy(), vn.float().numpy(), slots.numpy())
    ref = oracle.paged_decode_attention(w.q, k2, v2, w.block_table, ctx, w.scale)
    assert_parity(out.cpu(), ref, "write + attend")
    assert torch.equal(kd.cpu().view(torch.int16), torch.from_numpy(
        np.asarray(k2, dtype=np.float32)).to(torch.bfloat16).view(torch.int16))
