"""Helpers shared by the GPU tests: run the HIP path on a workload and compare
its BF16 output with the FP64 oracle."""

import sys

import numpy as np
import torch

import oracle

# Accuracy gate on BF16 outputs against the FP64 oracle, over all B*Hq*D values.
GATE_MAX_ABS = 2e-2
GATE_MEAN_ABS = 2e-3


def announce(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(w, dev="cuda:0"):
    return dict(q=w.q.to(dev), k_cache=w.k_cache.to(dev), v_cache=w.v_cache.to(dev),
                block_table=w.block_table.to(dev), context_lens=w.context_lens.to(dev))


def run_gpu(w, split_pages=0, scale=None, dev="cuda:0", tensors=None):
    from paged_gqa_attention_amd import pagedattn as pa
    t = tensors if tensors is not None else to_device(w, dev)
    out = pa.pa_decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                       scale=w.scale if scale is None else scale, split_pages=split_pages)
    torch.cuda.synchronize()
    return out.cpu()


def run_oracle(w, scale=None):
    return oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table,
                                         w.context_lens, w.scale if scale is None else scale)


def errors(gpu_bf16: torch.Tensor, ref: np.ndarray):
    g = gpu_bf16.float().numpy().astype(np.float64)
    d = np.abs(g - ref)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(d.max()), float(d.mean()), rel


def assert_parity(gpu_bf16, ref, what=""):
    g = gpu_bf16.float().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    mx, mean, rel = errors(gpu_bf16, ref)
    announce(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")
    assert mx <= GATE_MAX_ABS, f"{what}: max-abs {mx}"
    assert mean <= GATE_MEAN_ABS, f"{what}: mean-abs {mean}"
    return mx, mean, rel
