"""GPU parity of decode attention over FP8-E4M3 pools (pa_decode_fp8)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import announce, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from paged_gqa_attention_amd import pagedattn  # noqa: F401


def run_fp8(w, f, split_pages=0, scale=None):
    from paged_gqa_attention_amd import pagedattn as pa
    dev = "cuda:0"
    out = pa.pa_decode_fp8(w.q.to(dev), f.k_codes.to(dev), f.v_codes.to(dev), f.k_scale,
                           f.v_scale, w.block_table.to(dev), w.context_lens.to(dev),
                           scale=w.scale if scale is None else scale, split_pages=split_pages)
    torch.cuda.synchronize()
    return out.cpu()


def oracle_fp8(w, f, scale=None):
    return oracle.paged_decode_attention_fp8(w.q, f.k_codes, f.v_codes, f.k_scale, f.v_scale,
                                             w.block_table, w.context_lens,
                                             w.scale if scale is None else scale)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_fp8_standard_workloads(cfg):
    announce(f"fp8 workload {cfg}")
    w = workloads.config(cfg)
    f = workloads.quantize_fp8(w)
    assert_parity(run_fp8(w, f), oracle_fp8(w, f), f"fp8 config{cfg}")


@pytest.mark.parametrize("split_pages", [1, 3, 8])
def test_fp8_edges_and_splits(split_pages):
    ctx = [0, 1, 127, 128, 129, 2051, 4096]
    announce(f"fp8 edges split {split_pages}")
    w = workloads.build(len(ctx), 40, 8, 128, ctx, seed=17, max_pages=32, pool="packed")
    w = workloads.poison_unused(workloads.fill_unused_table(w, -1))
    f = workloads.quantize_fp8(w)
    out = run_fp8(w, f, split_pages=split_pages)
    assert torch.all(out[0] == 0)
    assert_parity(out, oracle_fp8(w, f), f"fp8 edges sp{split_pages}")


@pytest.mark.parametrize("D,G", [(128, 1), (128, 8), (256, 8), (256, 12), (128, 16)])
def test_fp8_shapes(D, G):
    ctx = [1, 300, 1000]
    w = workloads.build(3, 2 * G, 2, D, ctx, seed=G + D, max_pages=8, pool="packed")
    f = workloads.quantize_fp8(w)
    assert_parity(run_fp8(w, f), oracle_fp8(w, f), f"fp8 D{D} G{G}")


def test_fp8_every_v_code_through_context_one():
    # 254 finite codes laid out in the V rows of 32 one-token sequences; with
    # v_scale 1 the output of every query head is exactly that row's value
    announce("fp8 all V codes")
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    B, Hkv, D = 2, 1, 128
    w = workloads.build(B, 4, Hkv, D, [1, 1], seed=3, max_pages=1, pool="permutation")
    f = workloads.quantize_fp8(w)
    v = f.v_codes.clone()
    for b in range(B):
        page = int(w.block_table[b, 0])
        v[page, 0, 0] = torch.from_numpy(codes[b * D:(b + 1) * D] if b * D + D <= len(codes)
                                         else np.resize(codes[b * D:], D))
    f = workloads.Fp8Pools(f.k_codes, v, f.k_scale, 1.0)
    out = run_fp8(w, f)
    ref = oracle_fp8(w, f)
    assert np.array_equal(out.float().numpy().astype(np.float64), ref)


def test_fp8_every_k_code():
    # K rows cycle through all finite codes; q is one-hot so each logit is one
    # code's value: checks the K decode of every code against the oracle
    announce("fp8 all K codes")
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = 254
    w = workloads.build(1, 5, 1, 128, [n], seed=4, max_pages=2, pool="permutation")
    f = workloads.quantize_fp8(w)
    k = f.k_codes.clone()
    for t in range(n):
        page = int(w.block_table[0, t // 128])
        k[page, t % 128, 0] = torch.from_numpy(np.roll(codes, t)[:128])
    q = torch.zeros_like(w.q)
    q[0, :, 0] = 1.0          # logits = code value of dim 0 (times scales)
    q[0, 1, 5] = 0.5
    w.q = q
    f = workloads.Fp8Pools(k, f.v_codes, 0.03, f.v_scale)
    assert_parity(run_fp8(w, f), oracle_fp8(w, f), "fp8 all K codes")


def test_fp8_nan_code_in_a_read_slot_gives_nan_rows():
    w = workloads.build(2, 10, 2, 128, [50, 50], seed=5, max_pages=1, pool="permutation")
    f = workloads.quantize_fp8(w)
    k = f.k_codes.clone()
    k[int(w.block_table[1, 0]), 7, 1, 3] = 0x7F      # sequence 1, KV head 1
    out = run_fp8(w, workloads.Fp8Pools(k, f.v_codes, f.k_scale, f.v_scale))
    assert torch.isnan(out[1, 5:10].float()).all()
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[1, :5].float()).all()
