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


# ---- FP8-E4M3 pools ------------------------------------------------------------

def _codes_np(t):
    return t.contiguous().cpu().numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0137, 3.3e-3, 1e-30, 7.5e20, 2.0 ** -6])
def test_write_fp8_every_bf16_value(scale):
    # all 65536 BF16 bit patterns (zeros, subnormals, normals, infinities, NaNs)
    # through the kernel's division and conversion, compared code for code
    from paged_gqa_attention_amd import pagedattn as pa
    announce(f"kv write fp8: every bf16 value, scale {scale}")
    Hkv, D = 8, 128
    allv = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    kn = allv.reshape(64, Hkv, D)
    vn = allv.flip(0).reshape(64, Hkv, D).contiguous()
    slots = torch.arange(64, dtype=torch.int32) * 2          # every other slot of one page
    kc = torch.full((1, 128, Hkv, D), 0x5A, dtype=torch.uint8)
    vc = torch.full((1, 128, Hkv, D), 0xA5, dtype=torch.uint8)
    kd, vd = kc.cuda(), vc.cuda()
    pa.pa_kv_write_fp8(kn.cuda(), vn.cuda(), scale, 0.5 * scale, slots.cuda(), kd, vd)
    torch.cuda.synchronize()
    rk, rv = oracle.paged_kv_write_fp8(kc.numpy(), vc.numpy(), kn, vn, np.float32(scale),
                                       np.float32(0.5 * scale), slots.numpy())
    gk, gv = _codes_np(kd), _codes_np(vd)
    bad = np.nonzero(gk != rk)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"K code {gk[i]:#x} vs oracle {rk[i]:#x} at {i}, {bad[0].size} differ")
    assert np.array_equal(gv, rv)


@pytest.mark.parametrize("Hkv,D,T", [(8, 128, 16), (8, 128, 3000), (2, 256, 257), (1, 8, 5)])
def test_write_fp8_slots(Hkv, D, T):
    announce(f"kv write fp8 Hkv={Hkv} D={D} T={T}")
    from paged_gqa_attention_amd import pagedattn as pa
    N, P = 40, 128
    gen = torch.Generator().manual_seed(T + D + 1)
    kc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, dtype=torch.uint8)
    vc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, dtype=torch.uint8)
    kn = (3 * torch.randn(T, Hkv, D, generator=gen)).to(torch.bfloat16)
    vn = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
    slots = torch.randperm(N * P, generator=gen)[:T].to(torch.int32)
    slots[::7] = -1
    slots[3::11] = N * P + 5
    kd, vd = kc.cuda(), vc.cuda()
    pa.pa_kv_write_fp8(kn.cuda(), vn.cuda(), 0.021, 0.0078125, slots.cuda(), kd, vd)
    torch.cuda.synchronize()
    rk, rv = oracle.paged_kv_write_fp8(kc.numpy(), vc.numpy(), kn, vn, np.float32(0.021),
                                       np.float32(0.0078125), slots.numpy())
    assert np.array_equal(_codes_np(kd), rk)
    assert np.array_equal(_codes_np(vd), rv)


def test_fp8_write_then_attend():
    # a decode step over FP8 pools: quantise-write every sequence's new token,
    # then pa_decode_fp8 over ctx tokens, against the oracle doing the same
    announce("fp8 decode step: write + attend")
    from paged_gqa_attention_amd import pagedattn as pa
    w = workloads.config(2)
    f = workloads.quantize_fp8(w)
    B, Hkv, D = 16, 8, 128
    gen = torch.Generator().manual_seed(78)
    kn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    ctx = w.context_lens
    slots = torch.tensor([int(w.block_table[b, (int(c) - 1) // 128]) * 128 + (int(c) - 1) % 128
                          for b, c in enumerate(ctx)], dtype=torch.int32)
    dev = "cuda:0"
    kd, vd = f.k_codes.to(dev), f.v_codes.to(dev)
    pa.pa_kv_write_fp8(kn.to(dev), vn.to(dev), f.k_scale, f.v_scale, slots.to(dev), kd, vd)
    out = pa.pa_decode_fp8(w.q.to(dev), kd, vd, f.k_scale, f.v_scale, w.block_table.to(dev),
                           ctx.to(dev), scale=w.scale)
    torch.cuda.synchronize()
    k2, v2 = oracle.paged_kv_write_fp8(f.k_codes.numpy(), f.v_codes.numpy(), kn, vn,
                                       np.float32(f.k_scale), np.float32(f.v_scale), slots.numpy())
    assert np.array_equal(_codes_np(kd), k2) and np.array_equal(_codes_np(vd), v2)
    ref = oracle.paged_decode_attention_fp8(w.q, k2, v2, f.k_scale, f.v_scale, w.block_table, ctx,
                                            w.scale)
    assert_parity(out.cpu(), ref, "fp8 write + attend")
