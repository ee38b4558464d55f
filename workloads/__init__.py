"""Seeded synthetic inputs for paged GQA decode attention.

This module only draws inputs: context lengths, page-pool permutations, block
tables and BF16 q/K/V values. It holds none of the attention arithmetic, and it
is the one module that both the HIP-path tests and the oracle-side tests use,
so that both sides see identical bits.

Recipe (shared by every workload)
---------------------------------
* One CPU ``torch.Generator`` seeded with ``seed``; draws in the order
  context lengths, pool permutation, q, K, V.
* q, K and V are FP32 standard normal draws rounded to BF16 (round to nearest
  even, ``Tensor.to(torch.bfloat16)``), so the oracle can widen them exactly.
* The page pool is [num_pages, page_size, Hkv, D], the [page, token, kv_head,
  dim] order of the "Qwen3-14B" pypto-lib page ("decode_fwd" section), with
  128-token pages ("Deployment configuration" table).
* ``pool="permutation"``: the block table is a random permutation of all
  ``num_pages`` pages, reshaped to [B, W] (every entry valid; entries past a
  sequence's last page are never read).
* ``pool="packed"``: the pool has exactly sum(ceil(ctx/P)) pages; sequence b
  takes a consecutive chunk of a random permutation of them; unused entries
  are -1 (the -1 padding the orcarouter page mentions).
* ``scale`` defaults to the FP32 value of 1/sqrt(D) ("Qwen 3", TensorSharp
  docs, section 3: Q is multiplied by 1/sqrt(headDim)).

``quantize_fp8`` prepares FP8-E4M3 pools (codes plus one FP32 scale per
tensor) from a workload's BF16 pools; both sides then read the same codes.

The five standard workloads follow the decode shapes of the pages: Qwen3-14B's
40 query heads over 8 KV heads at head_dim 128, contexts up to 4096, and the
(16, 2) head_dim-256 local head shape the orcarouter page lists.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

PAGE_SIZE = 128
MAX_CONTEXT = 4096


@dataclass
class Workload:
    """One decode-attention call's inputs (CPU tensors)."""

    name: str
    q: torch.Tensor             # bf16 [B, Hq, D]
    k_cache: torch.Tensor       # bf16 [N, P, Hkv, D]
    v_cache: torch.Tensor       # bf16 [N, P, Hkv, D]
    block_table: torch.Tensor   # int32 [B, W]
    context_lens: torch.Tensor  # int32 [B]
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def page_size(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self) -> int:
        """K+V bytes a call must read: sum(ctx) * Hkv * D * 2 tensors * 2 B."""
        return int(self.context_lens.to(torch.int64).sum()) * self.num_kv_heads * self.head_dim * 4


def _bf16_normal(shape, gen) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def build(B: int, Hq: int, Hkv: int, D: int, ctx: Sequence[int], *, seed: int,
          page_size: int = PAGE_SIZE, max_pages: Optional[int] = None,
          pool: str = "permutation", num_pages: Optional[int] = None,
          scale: Optional[float] = None, name: str = "custom",
          gen: Optional[torch.Generator] = None) -> Workload:
    """Build a workload for the given context lengths.

    ``gen`` continues an existing generator (after the caller drew the context
    lengths from it); otherwise a fresh one is seeded with ``seed``.
    """
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    ctx_t = torch.as_tensor(list(ctx), dtype=torch.int32)
    assert ctx_t.numel() == B
    npages = [-(-int(c) // page_size) for c in ctx_t.tolist()]
    if max_pages is None:
        max_pages = max(1, max(npages) if npages else 1)
    assert all(n <= max_pages for n in npages), "context longer than the block table row"
    if pool == "permutation":
        if num_pages is None:
            num_pages = B * max_pages
        assert num_pages >= B * max_pages
        perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
        block_table = perm[: B * max_pages].reshape(B, max_pages).clone()
    elif pool == "packed":
        total = sum(npages)
        num_pages = max(1, total) if num_pages is None else num_pages
        assert num_pages >= total
        perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
        block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(npages):
            block_table[b, :n] = perm[off: off + n]
            off += n
    else:
        raise ValueError(pool)
    q = _bf16_normal((B, Hq, D), gen)
    k_cache = _bf16_normal((num_pages, page_size, Hkv, D), gen)
    v_cache = _bf16_normal((num_pages, page_size, Hkv, D), gen)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    return Workload(name, q, k_cache, v_cache, block_table, ctx_t, scale,
                    meta={"seed": seed, "pool": pool})


# The five standard workloads --------------------------------------------------

CONFIG_DESCRIPTIONS = {
    1: "single-layer paged GQA decode: B=2, ctx {1,130}, Hq=40, Hkv=8, D=128, 4-page pool",
    2: "Qwen3-14B decode layer attention: B=16, ctx U[1,4096], Hq=40, Hkv=8, D=128, 512-page shuffled pool",
    3: "bandwidth stress: B=16, ctx 4096, Hq=40, Hkv=8, D=128, 40 layers' caches called back to back",
    4: "large ragged batch: B=256, ctx lognormal(6.5,1) clipped to [1,4096], Hq=40, Hkv=8, D=128, packed pool",
    5: "wide-head GQA: B=32, Hq=16, Hkv=2, D=256, ctx U[256,4096], 1024-page shuffled pool, scale 1/16",
}

CONFIG_SHAPES = {
    1: dict(B=2, Hq=40, Hkv=8, D=128),
    2: dict(B=16, Hq=40, Hkv=8, D=128),
    3: dict(B=16, Hq=40, Hkv=8, D=128),
    4: dict(B=256, Hq=40, Hkv=8, D=128),
    5: dict(B=32, Hq=16, Hkv=2, D=256),
}

CONFIG3_LAYERS = 40


def config(i: int) -> Workload:
    """Standard workload ``i`` (1..5) with seed 1000 + i.

    For workload 3 this is layer 0 of the 40; the other layers share its block
    table and context lengths and only differ in q/K/V values.
    """
    seed = 1000 + i
    gen = torch.Generator().manual_seed(seed)
    s = CONFIG_SHAPES[i]
    name = f"config{i}"
    if i == 1:
        ctx = [1, 130]
        # pool of 4 pages, block table = a permutation of them viewed as [2, 2]
        return build(2, 40, 8, 128, ctx, seed=seed, gen=gen, max_pages=2,
                     pool="permutation", num_pages=4, name=name)
    if i == 2:
        ctx = torch.randint(1, MAX_CONTEXT + 1, (16,), generator=gen).tolist()
        return build(16, 40, 8, 128, ctx, seed=seed, gen=gen, max_pages=32,
                     pool="permutation", num_pages=512, name=name)
    if i == 3:
        ctx = [MAX_CONTEXT] * 16
        return build(16, 40, 8, 128, ctx, seed=seed, gen=gen, max_pages=32,
                     pool="permutation", num_pages=512, name=name)
    if i == 4:
        z = torch.randn(256, generator=gen, dtype=torch.float64)
        ctx = torch.clamp(torch.round(torch.exp(6.5 + z)), 1, MAX_CONTEXT).to(torch.int32).tolist()
        return build(256, 40, 8, 128, ctx, seed=seed, gen=gen, max_pages=32,
                     pool="packed", name=name)
    if i == 5:
        ctx = torch.randint(256, MAX_CONTEXT + 1, (32,), generator=gen).tolist()
        return build(32, 16, 2, 256, ctx, seed=seed, gen=gen, max_pages=32,
                     pool="permutation", num_pages=1024, name=name,
                     scale=float(torch.tensor(1.0 / 16.0, dtype=torch.float32)))
    raise ValueError(f"no standard workload {i}")


def poison_unused(w: Workload, value: float = float("nan")) -> Workload:
    """Fill every pool slot that no sequence reads with ``value`` (NaN default).

    Works for decode (``Workload``) and multi-query (``MqWorkload``) inputs.

    The tail slots of each sequence's last page and every page no sequence
    uses are overwritten; slots that some sequence reads are left alone.
    """
    N, P = int(w.k_cache.shape[0]), int(w.k_cache.shape[1])
    used = torch.zeros(N, P, dtype=torch.bool)
    for b in range(int(w.context_lens.numel())):
        n = int(w.context_lens[b])
        for j in range(-(-n // P)):
            page = int(w.block_table[b, j])
            valid = min(P, n - j * P)
            used[page, :valid] = True
    mask = (~used)[:, :, None, None].expand_as(w.k_cache)
    k = w.k_cache.clone()
    v = w.v_cache.clone()
    k[mask] = value
    v[mask] = value
    return dataclasses.replace(w, name=w.name + "+poison", k_cache=k, v_cache=v)


def fill_unused_table(w: Workload, value: int = -1) -> Workload:
    """Set every block-table entry past ceil(ctx/P) to ``value``."""
    bt = w.block_table.clone()
    P = w.page_size
    for b in range(w.batch):
        n = int(w.context_lens[b])
        bt[b, -(-n // P):] = value
    return Workload(w.name + f"+table{value}", w.q, w.k_cache, w.v_cache, bt, w.context_lens, w.scale, dict(w.meta))


FP8_E4M3_MAX = 448.0


@dataclass
class Fp8Pools:
    """FP8-E4M3 K/V pools (raw bytes) with per-tensor FP32 scales."""
    k_codes: torch.Tensor   # uint8 [N, P, Hkv, D]
    v_codes: torch.Tensor   # uint8 [N, P, Hkv, D]
    k_scale: float
    v_scale: float


def quantize_fp8(w: Workload) -> Fp8Pools:
    """Per-tensor FP8-E4M3 quantisation of a workload's K and V pools.

    scale = max|x| / 448 in FP32 (448 is the largest E4M3 value); codes are
    x / scale rounded to the nearest E4M3 value by torch's conversion, after
    clamping to +-448. NaN slots (poison) stay NaN codes.
    """
    def one(x):
        xf = x.float()
        finite = xf[torch.isfinite(xf)]
        amax = float(finite.abs().max()) if finite.numel() else 1.0
        scale = float(torch.tensor(max(amax, 1e-30) / FP8_E4M3_MAX, dtype=torch.float32))
        y = torch.clamp(xf / scale, -FP8_E4M3_MAX, FP8_E4M3_MAX)
        y = torch.where(torch.isnan(xf), xf, y)
        return y.to(torch.float8_e4m3fn).view(torch.uint8), scale
    kc, ks = one(w.k_cache)
    vc, vs = one(w.v_cache)
    return Fp8Pools(kc, vc, ks, vs)


# Multi-query (chunked prefill / multi-token decode) inputs --------------------

@dataclass
class MqWorkload:
    """One multi-query call's inputs (CPU tensors).

    q packs the query tokens of all sequences token-major: sequence b owns rows
    query_start[b] .. query_start[b+1]-1, the last Lq_b of its ctx_b cached
    tokens.
    """

    name: str
    q: torch.Tensor             # bf16 [T, Hq, D]
    k_cache: torch.Tensor       # bf16 [N, P, Hkv, D]
    v_cache: torch.Tensor       # bf16 [N, P, Hkv, D]
    block_table: torch.Tensor   # int32 [B, W]
    context_lens: torch.Tensor  # int32 [B]
    query_start: torch.Tensor   # int32 [B + 1]
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def max_query_len(self) -> int:
        d = self.query_start[1:] - self.query_start[:-1]
        return max(1, int(d.max())) if d.numel() else 1

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    def kv_bytes(self) -> int:
        """K+V bytes the call must read at least once: sum(ctx) * Hkv * D * 4."""
        return int(self.context_lens.to(torch.int64).sum()) * self.k_cache.shape[2] \
            * self.k_cache.shape[3] * 4

    def flops(self) -> int:
        """Multiply-adds x 2 of q.K and P.V over every row's visible tokens."""
        Hq, D = self.q.shape[1], self.q.shape[2]
        total = 0
        for b in range(self.context_lens.numel()):
            lq = int(self.query_start[b + 1] - self.query_start[b])
            ctx = int(self.context_lens[b])
            for i in range(lq):
                total += max(0, ctx - lq + i + 1)
        return total * Hq * D * 4


def build_mq(query_lens: Sequence[int], ctx: Sequence[int], Hq: int, Hkv: int, D: int, *,
             seed: int, max_pages: Optional[int] = None, pool: str = "permutation",
             num_pages: Optional[int] = None, scale: Optional[float] = None,
             name: str = "mq", gen: Optional[torch.Generator] = None) -> MqWorkload:
    """Build a multi-query workload: the cache as ``build`` draws it, then the
    T = sum(query_lens) packed query rows (BF16-rounded standard normals)."""
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    B = len(ctx)
    assert len(query_lens) == B
    w = build(B, Hq, Hkv, D, ctx, seed=seed, max_pages=max_pages, pool=pool,
              num_pages=num_pages, scale=scale, name=name, gen=gen)
    T = int(sum(query_lens))
    q = _bf16_normal((T, Hq, D), gen)
    qs = [0]
    for n in query_lens:
        qs.append(qs[-1] + int(n))
    return MqWorkload(name, q, w.k_cache, w.v_cache, w.block_table, w.context_lens,
                      torch.tensor(qs, dtype=torch.int32), w.scale,
                      meta={"seed": seed, "pool": pool})


MQ_DESCRIPTIONS = {
    "mtp4": "multi-token decode: B=16, 4 query tokens each, ctx 4096, Hq=40, Hkv=8, D=128, "
            "512-page shuffled pool",
    "prefill512": "chunked prefill: B=4, 512-token chunks ending at ctx U[512,4096], Hq=40, Hkv=8, "
                  "D=128, 128-page shuffled pool",
    "wide257": "wide-head prefill: B=4, 257 query tokens each, ctx U[257,4096], Hq=16, Hkv=2, "
               "D=256, 128-page shuffled pool, scale 1/16",
}


def mq_config(name: str) -> MqWorkload:
    """Standard multi-query workloads (seeded by name)."""
    seeds = {"mtp4": 2001, "prefill512": 2002, "wide257": 2003}
    seed = seeds[name]
    gen = torch.Generator().manual_seed(seed)
    if name == "mtp4":
        return build_mq([4] * 16, [MAX_CONTEXT] * 16, 40, 8, 128, seed=seed, gen=gen,
                        max_pages=32, num_pages=512, name=name)
    if name == "prefill512":
        ctx = torch.randint(512, MAX_CONTEXT + 1, (4,), generator=gen).tolist()
        return build_mq([512] * 4, ctx, 40, 8, 128, seed=seed, gen=gen, max_pages=32,
                        num_pages=128, name=name)
    if name == "wide257":
        ctx = torch.randint(257, MAX_CONTEXT + 1, (4,), generator=gen).tolist()
        return build_mq([257] * 4, ctx, 16, 2, 256, seed=seed, gen=gen, max_pages=32,
                        num_pages=128, name=name,
                        scale=float(torch.tensor(1.0 / 16.0, dtype=torch.float32)))
    raise ValueError(name)
