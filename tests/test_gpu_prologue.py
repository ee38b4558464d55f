"""GPU parity of the attention prologue (pa_attention_prologue): per-head
RMSNorm of q and k, NeoX RoPE, and the KV write, against the FP64 oracle.

Tolerance (derived): the kernel computes in FP32 (angles in FP64) and rounds
q and K to BF16 (nearest even), so each element may differ from the FP64
value by the BF16 rounding, at most 2^-8 * |value|, plus the FP32 error of the
norm and the rotation (relative ~1e-6 of the head's largest value, < 1e-4
here). Gate per element: |gpu - oracle| <= 2^-8 * |oracle| + 1e-4. V is a copy:
bit-exact. Cache rows no token writes must be untouched (bit-exact).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import announce, assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_REL = 2.0 ** -8
TOL_ABS = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from paged_gqa_attention_amd import pagedattn  # noqa: F401


def make_inputs(T, Hq, Hkv, D, N, seed, positions=None, slots=None, w_scale=1.0):
    gen = torch.Generator().manual_seed(seed)
    bf = lambda *s: torch.randn(*s, generator=gen).to(torch.bfloat16)
    q, k, v = bf(T, Hq, D), bf(T, Hkv, D), bf(T, Hkv, D)
    wq = (1.0 + w_scale * torch.randn(D, generator=gen)).to(torch.bfloat16)
    wk = (1.0 + w_scale * torch.randn(D, generator=gen)).to(torch.bfloat16)
    kc, vc = bf(N, 128, Hkv, D), bf(N, 128, Hkv, D)
    if positions is None:
        positions = torch.randint(0, 4096, (T,), generator=gen)
    if slots is None:
        slots = torch.randperm(N * 128, generator=gen)[:T]
    return dict(q=q, k=k, v=v, wq=wq, wk=wk, kc=kc, vc=vc,
                pos=torch.as_tensor(positions, dtype=torch.int32),
                slots=torch.as_tensor(slots, dtype=torch.int32))


def run_gpu(x, eps=1e-6, base=1e6, scale=1.0, in_place=False):
    from paged_gqa_attention_amd import pagedattn as pa
    g = {n: t.to(DEV) for n, t in x.items()}
    out = g["q"] if in_place else None
    qo = pa.pa_attention_prologue(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["pos"], g["slots"],
                                  g["kc"], g["vc"], eps=eps, rope_base=base, rope_scale=scale,
                                  q_out=out)
    torch.cuda.synchronize()
    return qo.cpu(), g["kc"].cpu(), g["vc"].cpu()


def run_oracle(x, eps=1e-6, base=1e6, scale=1.0):
    return oracle.attention_prologue(x["q"], x["k"], x["v"], x["wq"], x["wk"], x["pos"],
                                     x["slots"], np.float32(eps), np.float32(base),
                                     np.float32(scale), x["kc"], x["vc"])


def assert_close(gpu, ref, what):
    g = gpu.float().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - ref)
    bound = TOL_REL * np.abs(ref) + TOL_ABS
    worst = float(np.max(err / bound))
    announce(f"{what}: max-abs {err.max():.3e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, what


def check(x, eps=1e-6, base=1e6, scale=1.0, in_place=False, what=""):
    qo, kc, vc = run_gpu(x, eps, base, scale, in_place)
    rq, rk, rv = run_oracle(x, eps, base, scale)
    assert_close(qo, rq, f"{what} q")
    slots = x["slots"].tolist()
    N = x["kc"].shape[0]
    written = np.zeros((N, 128), bool)
    for s in slots:
        if 0 <= s < N * 128:
            written[s // 128, s % 128] = True
    assert_close(kc[torch.from_numpy(written)], rk[written], f"{what} K rows")
    # V: bit-exact copy; everything not written: untouched
    assert torch.equal(vc.view(torch.int16)[torch.from_numpy(written)],
                       torch.from_numpy(rv[written]).to(torch.bfloat16).view(torch.int16))
    nw = torch.from_numpy(~written)
    assert torch.equal(kc[nw].view(torch.int16), x["kc"][nw].view(torch.int16))
    assert torch.equal(vc[nw].view(torch.int16), x["vc"][nw].view(torch.int16))
    return qo, kc, vc


def test_decode_step_qwen_shape():
    announce("prologue decode step 16 tokens 40/8/128")
    check(make_inputs(16, 40, 8, 128, 512, seed=1), what="decode step")


def test_prefill_chunk_sequential_positions():
    announce("prologue prefill chunk 2048 tokens")
    T = 2048
    x = make_inputs(T, 40, 8, 128, 64, seed=2, positions=np.arange(1000, 1000 + T),
                    slots=np.arange(T) + 3 * 128)
    check(x, what="prefill chunk")


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 256), (24, 2, 256), (3, 1, 256), (8, 8, 128),
                                      (5, 1, 128), (64, 4, 128)])
def test_head_shapes(Hq, Hkv, D):
    announce(f"prologue heads {Hq}/{Hkv} D{D}")
    check(make_inputs(37, Hq, Hkv, D, 40, seed=Hq + D), what=f"{Hq}/{Hkv}/{D}")


@pytest.mark.parametrize("eps,base,scale", [(1e-6, 1e6, 1.0), (1e-5, 1e4, 1.0), (1e-6, 1e6, 4.0),
                                            (0.0, 5e5, 0.5), (0.1, 1e6, 1.0)])
def test_norm_and_rope_parameters(eps, base, scale):
    announce(f"prologue eps {eps} base {base} scale {scale}")
    check(make_inputs(24, 40, 8, 128, 16, seed=3), eps=eps, base=base, scale=scale,
          what=f"params {eps},{base},{scale}")


def test_large_positions_need_fp64_angles():
    # positions near 2^27 (the largest a 2^20-page table can address): an FP32
    # angle would be off by radians at the high frequencies
    announce("prologue large positions")
    pos = np.array([0, 1, 4095, 65536, 1 << 20, (1 << 27) - 1, 123456789, 99999999])
    check(make_inputs(8, 40, 8, 128, 4, seed=4, positions=pos), what="large positions")


def test_padding_and_out_of_pool_slots_write_nothing():
    announce("prologue padding slots")
    N = 4
    slots = np.array([5, -1, 130, N * 128, -7, 511, N * 128 + 1000, 0])
    check(make_inputs(8, 40, 8, 128, N, seed=5, slots=slots), what="padding")


def test_in_place_q():
    announce("prologue in place")
    x = make_inputs(33, 40, 8, 128, 8, seed=6)
    check(x, in_place=True, what="in place")


def test_position_zero_is_the_normalised_input():
    # theta = 0: RoPE is the identity, so q_out = bf16(RMSNorm(q)) exactly as
    # the FP32 norm rounds
    announce("prologue position 0")
    x = make_inputs(6, 40, 8, 128, 2, seed=7, positions=np.zeros(6))
    qo, _, _ = check(x, what="position 0")
    ref = oracle.rms_norm_heads(x["q"], x["wq"], np.float32(1e-6))
    assert_close(qo, ref, "position 0 vs norm only")


def test_decode_step_end_to_end():
    # prologue writes the new token's K/V at slot ctx-1, then decode attention
    # reads it together with the older tokens; compared with the oracle's
    # prologue followed by the oracle's decode attention
    from paged_gqa_attention_amd import pagedattn as pa
    announce("prologue + decode end to end")
    B, Hq, Hkv, D = 4, 40, 8, 128
    ctx = [1, 130, 1000, 4096]
    w = workloads.build(B, Hq, Hkv, D, ctx, seed=8, max_pages=32, pool="permutation")
    bt = w.block_table
    slots = [int(bt[b, (c - 1) // 128]) * 128 + (c - 1) % 128 for b, c in enumerate(ctx)]
    gen = torch.Generator().manual_seed(9)
    bf = lambda *s: torch.randn(*s, generator=gen).to(torch.bfloat16)
    q_raw, k_raw, v_raw = bf(B, Hq, D), bf(B, Hkv, D), bf(B, Hkv, D)
    wq = (1 + 0.2 * torch.randn(D, generator=gen)).to(torch.bfloat16)
    wk = (1 + 0.2 * torch.randn(D, generator=gen)).to(torch.bfloat16)
    pos = torch.tensor([c - 1 for c in ctx], dtype=torch.int32)
    sl = torch.tensor(slots, dtype=torch.int32)
    g = dict(q=q_raw.to(DEV), k=k_raw.to(DEV), v=v_raw.to(DEV), wq=wq.to(DEV), wk=wk.to(DEV),
             pos=pos.to(DEV), sl=sl.to(DEV), kc=w.k_cache.to(DEV), vc=w.v_cache.to(DEV),
             bt=bt.to(DEV), ctx=w.context_lens.to(DEV))
    qo = pa.pa_attention_prologue(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["pos"], g["sl"],
                                  g["kc"], g["vc"])
    out = pa.pa_decode(qo, g["kc"], g["vc"], g["bt"], g["ctx"], scale=w.scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_prologue(q_raw, k_raw, v_raw, wq, wk, pos, sl, np.float32(1e-6),
                                           np.float32(1e6), np.float32(1.0), w.k_cache, w.v_cache)
    # the oracle's attention takes BF16 inputs: feed it the BF16-rounded prologue
    # outputs (what the cache and q hold), each checked against FP64 above
    rq16 = torch.from_numpy(rq).to(torch.bfloat16)
    rk16 = torch.from_numpy(rk).to(torch.bfloat16)
    rv16 = torch.from_numpy(rv).to(torch.bfloat16)
    assert_close(qo.cpu(), rq, "e2e q")
    ref = oracle.paged_decode_attention(rq16, rk16, rv16, bt, w.context_lens, w.scale)
    assert_parity(out.cpu(), ref, "prologue + decode")


# ---- FP8-E4M3 pools ------------------------------------------------------------
# K codes: the kernel's BF16 K row (within the gate above of the FP64 row)
# divided by k_scale and encoded, so the decoded value is within half an E4M3
# step (2^-4 relative, 2^-10 * k_scale absolute below the normal range) of that
# row: gate |code * k_scale - K_oracle| <= (2^-4 + 2^-8)|K| * 1.001 + 2^-10 k_scale
# + 1e-4. V codes: bit-exact (the division and encoding of the BF16 input are
# fixed). The K codes also equal pa_kv_write_fp8 of the BF16 prologue's own K
# rows, bit for bit (same rounding to BF16, same encoder).

def run_gpu_fp8(x, ks, vs, kc8, vc8, eps=1e-6, base=1e6, scale=1.0):
    from paged_gqa_attention_amd import pagedattn as pa
    g = {n: t.to(DEV) for n, t in x.items()}
    k8, v8 = kc8.to(DEV), vc8.to(DEV)
    qo = pa.pa_attention_prologue_fp8(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["pos"],
                                      g["slots"], ks, vs, k8, v8, eps=eps, rope_base=base,
                                      rope_scale=scale)
    torch.cuda.synchronize()
    return qo.cpu(), k8.cpu(), v8.cpu()


def check_fp8(x, ks, vs, what, eps=1e-6, base=1e6, scale=1.0):
    from paged_gqa_attention_amd import pagedattn as pa
    N, P, Hkv, D = x["kc"].shape
    gen = torch.Generator().manual_seed(5)
    kc8 = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, dtype=torch.uint8)
    vc8 = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, dtype=torch.uint8)
    qo, k8, v8 = run_gpu_fp8(x, ks, vs, kc8, vc8, eps, base, scale)
    rq, rk8, rv8 = oracle.attention_prologue_fp8(
        x["q"], x["k"], x["v"], x["wq"], x["wk"], x["pos"], x["slots"], np.float32(eps),
        np.float32(base), np.float32(scale), np.float32(ks), np.float32(vs), kc8.numpy(),
        vc8.numpy())
    assert_close(qo, rq, f"{what} q")
    written = np.zeros((N, P), bool)
    for s in x["slots"].tolist():
        if 0 <= s < N * P:
            written[s // P, s % P] = True
    assert np.array_equal(v8.numpy(), rv8), f"{what} V codes"
    assert np.array_equal(k8.numpy()[~written], kc8.numpy()[~written]), f"{what} untouched K"
    # K against the FP64 rotated rows (the oracle's BF16 prologue, unrounded)
    _, rk64, _ = run_oracle(x, eps, base, scale)
    dec = oracle.decode_fp8_e4m3(k8.numpy()[written]) * float(np.float32(ks))
    lim = 448.0 * float(np.float32(ks))                   # codes saturate at +-448
    ref = np.clip(rk64[written], -lim, lim)
    bound = (2.0 ** -4 + 2.0 ** -8) * np.abs(ref) * 1.001 + 2.0 ** -10 * ks + 1e-4
    err = np.abs(dec - ref)
    announce(f"{what} K codes: worst err/bound {float(np.max(err / bound)):.3f}, "
             f"{float(np.mean(k8.numpy()[written] == rk8[written])):.5f} equal to the oracle's")
    assert np.all(err <= bound), f"{what} K codes"
    # the same bits as the BF16 prologue followed by the FP8 KV write
    g = {n: t.to(DEV) for n, t in x.items()}
    pa.pa_attention_prologue(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["pos"], g["slots"],
                             g["kc"], g["vc"], eps=eps, rope_base=base, rope_scale=scale)
    k16 = torch.stack([g["kc"][s // P, s % P] for s in x["slots"].tolist() if 0 <= s < N * P]) \
        if written.any() else None
    if k16 is not None:
        sl = torch.tensor([s for s in x["slots"].tolist() if 0 <= s < N * P], dtype=torch.int32)
        k8b, v8b = kc8.to(DEV), vc8.to(DEV)
        vrows = torch.stack([x["v"][t] for t, s in enumerate(x["slots"].tolist())
                             if 0 <= s < N * P]).to(DEV)
        pa.pa_kv_write_fp8(k16.contiguous(), vrows.contiguous(), ks, vs, sl.to(DEV), k8b, v8b)
        torch.cuda.synchronize()
        assert torch.equal(k8b.cpu(), k8), f"{what}: prologue_fp8 != prologue + kv_write_fp8"


@pytest.mark.parametrize("Hq,Hkv,D,ks", [(40, 8, 128, 0.05), (16, 2, 256, 0.02), (8, 8, 128, 1.0)])
def test_fp8_prologue(Hq, Hkv, D, ks):
    announce(f"fp8 prologue {Hq}/{Hkv}/{D} k_scale {ks}")
    x = make_inputs(300, Hq, Hkv, D, 8, seed=Hq + D + 7)
    check_fp8(x, ks, 0.0137, f"fp8 prologue {Hq}/{Hkv}/{D}")


def test_fp8_prologue_padding_saturation_and_parameters():
    # padding and out-of-pool slots write nothing; a tiny k_scale saturates K
    # codes at +-448 (the bound then does not hold: checked separately)
    announce("fp8 prologue padding / parameters")
    x = make_inputs(20, 40, 8, 128, 4, seed=77, slots=[5, -1, 4 * 128, 7, -9] + list(range(8, 23)),
                    positions=[(1 << 27) - 1] + list(range(19)))
    check_fp8(x, 0.05, 0.02, "fp8 prologue params", eps=1e-5, base=1e4, scale=4.0)
    from paged_gqa_attention_amd import pagedattn as pa
    kc8 = torch.zeros(4, 128, 8, 128, dtype=torch.uint8)
    qo, k8, v8 = run_gpu_fp8(x, 1e-4, 1e-4, kc8, kc8.clone())
    codes = k8[0, 5].numpy()
    assert set(np.unique(codes & 0x7F).tolist()) <= set(range(0x7F))   # never NaN
    assert np.mean((codes & 0x7F) == 0x7E) > 0.9                        # saturated
