"""GPU parity of the fused decode step (pa_decode_step): the attention
prologue of each sequence's new token (QK-norm, NeoX RoPE, KV write) run by the
decode kernel itself, then decode attention. Reference: the oracle's prologue
followed by the oracle's decode attention over the BF16-rounded results.

Gates: attention outputs as every decode test (max-abs 2e-2, mean-abs 2e-3);
written K rows per element within 2^-8 |x| + 1e-4 of the oracle (BF16 rounding
plus FP32 norm and rotation, as for pa_attention_prologue); written V rows and
every other pool row bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import announce, assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from paged_gqa_attention_amd import pagedattn  # noqa: F401


def make_step(B, Hq, Hkv, D, ctx, seed, W=None, positions=None, pool="permutation"):
    w = workloads.build(B, Hq, Hkv, D, ctx, seed=seed, max_pages=W, pool=pool)
    gen = torch.Generator().manual_seed(seed + 1000)
    bf = lambda *s: torch.randn(*s, generator=gen).to(torch.bfloat16)
    q, k, v = bf(B, Hq, D), bf(B, Hkv, D), bf(B, Hkv, D)
    wq = (1 + 0.3 * torch.randn(D, generator=gen)).to(torch.bfloat16)
    wk = (1 + 0.3 * torch.randn(D, generator=gen)).to(torch.bfloat16)
    bt = w.block_table
    slots = [int(bt[b, (c - 1) // 128]) * 128 + (c - 1) % 128 if c > 0 else -1
             for b, c in enumerate(ctx)]
    pos = [c - 1 if c > 0 else 0 for c in ctx] if positions is None else positions
    return w, dict(q=q, k=k, v=v, wq=wq, wk=wk, pos=torch.tensor(pos, dtype=torch.int32),
                   slots=torch.tensor(slots, dtype=torch.int32))


def run_step(w, x, split_pages=0, eps=1e-6, base=1e6, rscale=1.0, slots=None):
    from paged_gqa_attention_amd import pagedattn as pa
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    sl = x["slots"] if slots is None else slots
    out = pa.pa_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["wq"].to(DEV),
                            x["wk"].to(DEV), x["pos"].to(DEV), sl.to(DEV), kc, vc,
                            w.block_table.to(DEV), w.context_lens.to(DEV), scale=w.scale,
                            eps=eps, rope_base=base, rope_scale=rscale, split_pages=split_pages)
    torch.cuda.synchronize()
    return out.cpu(), kc.cpu(), vc.cpu()


def reference(w, x, eps=1e-6, base=1e6, rscale=1.0):
    """Oracle prologue (FP64, caches written at the slots), then oracle decode
    over the BF16-rounded q and caches."""
    rq, rk, rv = oracle.attention_prologue(x["q"], x["k"], x["v"], x["wq"], x["wk"], x["pos"],
                                           x["slots"], np.float32(eps), np.float32(base),
                                           np.float32(rscale), w.k_cache, w.v_cache)
    q16 = torch.from_numpy(rq).to(torch.bfloat16)
    k16 = torch.from_numpy(rk).to(torch.bfloat16)
    v16 = torch.from_numpy(rv).to(torch.bfloat16)
    out = oracle.paged_decode_attention(q16, k16, v16, w.block_table, w.context_lens, w.scale)
    return out, rk, rv


def check_pools(w, x, kc, vc, rk, rv, what):
    N = w.k_cache.shape[0]
    written = np.zeros((N, 128), bool)
    for s in x["slots"].tolist():
        if 0 <= s < N * 128:
            written[s // 128, s % 128] = True
    m = torch.from_numpy(written)
    g = kc[m].float().numpy().astype(np.float64)
    ref = rk[written]
    assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4), f"{what}: K rows"
    assert torch.equal(vc[m].view(torch.int16),
                       torch.from_numpy(rv[written]).to(torch.bfloat16).view(torch.int16))
    assert torch.equal(kc[~m].view(torch.int16), w.k_cache[~m].view(torch.int16))
    assert torch.equal(vc[~m].view(torch.int16), w.v_cache[~m].view(torch.int16))


@pytest.mark.parametrize("split_pages", [0, 1, 3])
def test_decode_step_qwen_shape(split_pages):
    announce(f"decode step 40/8/128 sp{split_pages}")
    ctx = [1, 130, 1000, 4096, 129, 2048]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=31, W=32)
    out, kc, vc = run_step(w, x, split_pages)
    ref, rk, rv = reference(w, x)
    assert_parity(out, ref, f"decode step sp{split_pages}")
    check_pools(w, x, kc, vc, rk, rv, "decode step")


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 256), (24, 2, 256), (8, 8, 128), (16, 1, 128),
                                      (3, 1, 256)])
def test_decode_step_head_shapes(Hq, Hkv, D):
    announce(f"decode step {Hq}/{Hkv}/{D}")
    ctx = [17, 300, 777]
    w, x = make_step(len(ctx), Hq, Hkv, D, ctx, seed=Hq + D, W=8)
    out, kc, vc = run_step(w, x)
    ref, rk, rv = reference(w, x)
    assert_parity(out, ref, f"decode step {Hq}/{Hkv}/{D}")
    check_pools(w, x, kc, vc, rk, rv, f"decode step {Hq}/{Hkv}/{D}")


def test_decode_step_parameters_and_large_positions():
    # RoPE at large positions (FP64 frequencies and reduction), other norm and
    # rope parameters; positions need not equal ctx - 1
    announce("decode step large positions")
    ctx = [5, 200, 1000, 3000]
    pos = [(1 << 27) - 1, 123456789, 4095, 0]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=33, W=24, positions=pos)
    for eps, base, rs in ((1e-6, 1e6, 1.0), (1e-5, 1e4, 4.0), (0.0, 5e5, 0.5)):
        out, kc, vc = run_step(w, x, eps=eps, base=base, rscale=rs)
        ref, rk, rv = reference(w, x, eps=eps, base=base, rscale=rs)
        assert_parity(out, ref, f"decode step eps {eps} base {base} scale {rs}")
        check_pools(w, x, kc, vc, rk, rv, "decode step params")


def test_decode_step_empty_context_and_unwritten_slot():
    # ctx 0: zeros, nothing written. slot -1: nothing written, but attention
    # still sees the new token's K/V (taken from the fused prologue)
    announce("decode step ctx 0 and slot -1")
    ctx = [0, 300, 129]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=34, W=4)
    slots = x["slots"].clone()
    slots[2] = -1
    out, kc, vc = run_step(w, x, slots=slots)
    ref, rk, rv = reference(w, x)       # as if sequence 2's slot were written
    assert torch.all(out[0] == 0)
    assert_parity(out, ref, "decode step ctx 0 / slot -1")
    x2 = dict(x, slots=slots)
    check_pools(w, x2, kc, vc, rk, rv, "decode step slot -1")


def test_decode_step_matches_separate_prologue_and_decode():
    # the fused step against pa_attention_prologue followed by pa_decode on the
    # GPU: same math, angles computed differently (tolerance, not bits)
    from paged_gqa_attention_amd import pagedattn as pa
    announce("decode step vs separate kernels")
    ctx = [1, 257, 4096, 1500]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=35, W=32)
    fused, kcf, vcf = run_step(w, x)
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    qo = pa.pa_attention_prologue(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                                  x["wq"].to(DEV), x["wk"].to(DEV), x["pos"].to(DEV),
                                  x["slots"].to(DEV), kc, vc)
    sep = pa.pa_decode(qo, kc, vc, w.block_table.to(DEV), w.context_lens.to(DEV),
                       scale=w.scale).cpu()
    torch.cuda.synchronize()
    d = (fused.float() - sep.float()).abs()
    announce(f"  fused vs separate: max-abs {float(d.max()):.3e}")
    assert float(d.max()) <= 2e-2 and float(d.mean()) <= 2e-3
    assert torch.equal(vcf.view(torch.int16), vc.cpu().view(torch.int16))
    kd = (kcf.float() - kc.cpu().float()).abs()
    assert float(kd.max()) <= 2.0 ** -7 * float(kc.cpu().float().abs().max())


# ---- FP8-E4M3 pools (pa_decode_step_fp8) -----------------------------------------
# The new token's K (BF16 after norm and RoPE) and V are written as codes;
# attention reads the codes. Reference: the oracle's FP8 prologue (codes of the
# BF16-rounded FP64 K row) and its FP8 decode over the codes it wrote. The
# kernel's BF16 K row may differ from the oracle's by one BF16 step, so single
# K codes may differ by one E4M3 step: K codes are gated against the FP64 row
# (half a step, as for pa_attention_prologue_fp8), the attention output by the
# usual gate; V codes and untouched rows are bit-exact. K values past
# 448 * k_scale saturate (the reference is clipped there).

def run_step_fp8(w, x, f, split_pages=0, eps=1e-6, base=1e6, rscale=1.0):
    from paged_gqa_attention_amd import pagedattn as pa
    kc, vc = f.k_codes.to(DEV), f.v_codes.to(DEV)
    out = pa.pa_decode_step_fp8(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["wq"].to(DEV),
                                x["wk"].to(DEV), x["pos"].to(DEV), x["slots"].to(DEV), f.k_scale,
                                f.v_scale, kc, vc, w.block_table.to(DEV), w.context_lens.to(DEV),
                                scale=w.scale, eps=eps, rope_base=base, rope_scale=rscale,
                                split_pages=split_pages)
    torch.cuda.synchronize()
    return out.cpu(), kc.cpu(), vc.cpu()


def reference_fp8(w, x, f, eps=1e-6, base=1e6, rscale=1.0):
    rq, rk8, rv8 = oracle.attention_prologue_fp8(
        x["q"], x["k"], x["v"], x["wq"], x["wk"], x["pos"], x["slots"], np.float32(eps),
        np.float32(base), np.float32(rscale), np.float32(f.k_scale), np.float32(f.v_scale),
        f.k_codes.numpy(), f.v_codes.numpy())
    q16 = torch.from_numpy(rq).to(torch.bfloat16)
    out = oracle.paged_decode_attention_fp8(q16, rk8, rv8, f.k_scale, f.v_scale, w.block_table,
                                            w.context_lens, w.scale)
    return out, rk8, rv8


def check_pools_fp8(w, x, f, kc, vc, rv8, what, eps=1e-6, base=1e6, rscale=1.0):
    N = w.k_cache.shape[0]
    written = np.zeros((N, 128), bool)
    for s in x["slots"].tolist():
        if 0 <= s < N * 128:
            written[s // 128, s % 128] = True
    assert np.array_equal(vc.numpy(), rv8), f"{what}: V codes"
    assert np.array_equal(kc.numpy()[~written], f.k_codes.numpy()[~written]), f"{what}: K rows"
    _, rk64, _ = oracle.attention_prologue(x["q"], x["k"], x["v"], x["wq"], x["wk"], x["pos"],
                                           x["slots"], np.float32(eps), np.float32(base),
                                           np.float32(rscale), w.k_cache, w.v_cache)
    lim = 448.0 * float(np.float32(f.k_scale))           # codes saturate at +-448
    ref = np.clip(rk64[written], -lim, lim)
    dec = oracle.decode_fp8_e4m3(kc.numpy()[written]) * float(np.float32(f.k_scale))
    bound = (2.0 ** -4 + 2.0 ** -8) * np.abs(ref) * 1.001 + 2.0 ** -10 * f.k_scale + 1e-4
    assert np.all(np.abs(dec - ref) <= bound), f"{what}: new K codes"


@pytest.mark.parametrize("split_pages", [0, 1])
def test_decode_step_fp8_qwen_shape(split_pages):
    announce(f"decode step fp8 40/8/128 sp{split_pages}")
    ctx = [1, 130, 1000, 4096, 129, 2048]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=41, W=32)
    f = workloads.quantize_fp8(w)
    out, kc, vc = run_step_fp8(w, x, f, split_pages)
    ref, rk8, rv8 = reference_fp8(w, x, f)
    assert_parity(out, ref, f"decode step fp8 sp{split_pages}")
    check_pools_fp8(w, x, f, kc, vc, rv8, "decode step fp8")


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 256), (8, 8, 128), (3, 1, 256)])
def test_decode_step_fp8_head_shapes(Hq, Hkv, D):
    announce(f"decode step fp8 {Hq}/{Hkv}/{D}")
    ctx = [17, 300, 777]
    w, x = make_step(len(ctx), Hq, Hkv, D, ctx, seed=Hq + D + 3, W=8)
    f = workloads.quantize_fp8(w)
    out, kc, vc = run_step_fp8(w, x, f)
    ref, rk8, rv8 = reference_fp8(w, x, f)
    assert_parity(out, ref, f"decode step fp8 {Hq}/{Hkv}/{D}")
    check_pools_fp8(w, x, f, kc, vc, rv8, f"decode step fp8 {Hq}/{Hkv}/{D}")


def test_decode_step_fp8_parameters_and_empty_context():
    announce("decode step fp8 parameters, ctx 0")
    ctx = [0, 200, 1000, 3000]
    pos = [0, 123456789, 4095, (1 << 27) - 1]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=43, W=24, positions=pos)
    f = workloads.quantize_fp8(w)
    out, kc, vc = run_step_fp8(w, x, f, eps=1e-5, base=1e4, rscale=4.0)
    ref, rk8, rv8 = reference_fp8(w, x, f, eps=1e-5, base=1e4, rscale=4.0)
    assert torch.all(out[0] == 0)
    assert_parity(out, ref, "decode step fp8 params")
    check_pools_fp8(w, x, f, kc, vc, rv8, "decode step fp8 params", eps=1e-5, base=1e4, rscale=4.0)


def test_decode_step_fp8_matches_separate_kernels():
    # against pa_attention_prologue_fp8 then pa_decode_fp8 on the GPU
    from paged_gqa_attention_amd import pagedattn as pa
    announce("decode step fp8 vs separate kernels")
    ctx = [1, 257, 4096, 1500]
    w, x = make_step(len(ctx), 40, 8, 128, ctx, seed=45, W=32)
    f = workloads.quantize_fp8(w)
    fused, kcf, vcf = run_step_fp8(w, x, f)
    kc, vc = f.k_codes.to(DEV), f.v_codes.to(DEV)
    qo = pa.pa_attention_prologue_fp8(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                                      x["wq"].to(DEV), x["wk"].to(DEV), x["pos"].to(DEV),
                                      x["slots"].to(DEV), f.k_scale, f.v_scale, kc, vc)
    sep = pa.pa_decode_fp8(qo, kc, vc, f.k_scale, f.v_scale, w.block_table.to(DEV),
                           w.context_lens.to(DEV), scale=w.scale).cpu()
    torch.cuda.synchronize()
    d = (fused.float() - sep.float()).abs()
    announce(f"  fused vs separate: max-abs {float(d.max()):.3e}")
    assert float(d.max()) <= 2e-2 and float(d.mean()) <= 2e-3
    assert torch.equal(vcf, vc.cpu())
    a = oracle.decode_fp8_e4m3(kcf.numpy())
    b = oracle.decode_fp8_e4m3(kc.cpu().numpy())
    assert np.all(np.abs(a - b) <= 2.0 ** -3 * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -9)
