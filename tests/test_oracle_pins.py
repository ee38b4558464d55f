"""Pins for the FP64 oracle, each against something other than the oracle itself.

Every check here runs on the CPU. A plausible mistake in the oracle (a dropped
scale, a wrong KV-head mapping, a transposed operand, an off-by-one in the
context length, a wrong page or slot index) fails at least one of them; the
mutation tests at the end plant such mistakes in the oracle and assert that the
pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as oracle_decode
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _f64(t):
    return t.float().numpy().astype(np.float64)


def _tiny(seed=7, ctx=(0, 1, 4, 5, 11), Hq=6, Hkv=2, D=8, P=4, W=3, N=16, poison=True):
    gen = torch.Generator().manual_seed(seed)
    w = workloads.build(len(ctx), Hq, Hkv, D, ctx, seed=seed, gen=gen, page_size=P,
                        max_pages=W, pool="permutation", num_pages=N)
    w = workloads.fill_unused_table(w, -1)
    if poison:
        w = workloads.poison_unused(w)
    return w


# ---------------------------------------------------------------------------
# I1: a pure-Python scalar brute force with explicit flat-pool addressing
# ---------------------------------------------------------------------------

def _brute_force(w):
    """Scalar loops over the flat [page, token, kv_head, dim] byte order.

    Element (page, slot, h, d) of a pool is at ((page*P + slot)*Hkv + h)*D + d;
    token t of sequence b is in page block_table[b][t // P] at slot t % P.
    Query head hq reads KV head hq // G. Logits use math.fsum; weights math.exp.
    """
    B, Hq, D = w.q.shape
    N, P, Hkv, _ = w.k_cache.shape
    G = Hq // Hkv
    qf = w.q.float().flatten().tolist()
    kf = w.k_cache.float().flatten().tolist()
    vf = w.v_cache.float().flatten().tolist()
    bt = w.block_table.tolist()
    ctx = w.context_lens.tolist()
    scale = float(np.float32(w.scale))
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        n = ctx[b]
        if n == 0:
            continue
        for hq in range(Hq):
            h = hq // G
            qrow = qf[(b * Hq + hq) * D:(b * Hq + hq + 1) * D]
            bases = []
            for t in range(n):
                page = bt[b][t // P]
                slot = t % P
                bases.append(((page * P + slot) * Hkv + h) * D)
            logits = [scale * math.fsum(qrow[d] * kf[base + d] for d in range(D)) for base in bases]
            mx = max(logits)
            e = [math.exp(x - mx) for x in logits]
            Z = math.fsum(e)
            for d in range(D):
                out[b][hq][d] = math.fsum(e[t] * vf[bases[t] + d] for t in range(n)) / Z
    return np.array(out, dtype=np.float64)


def test_i1_brute_force_tiny():
    w = _tiny()
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    ref = _brute_force(w)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("Hq,Hkv,D,P,ctx", [
    (4, 4, 8, 4, (3, 9)),           # G = 1 (plain multi-head attention)
    (8, 1, 4, 2, (1, 2, 7)),        # G = 8 over one KV head
    (12, 1, 16, 8, (17, 8, 9)),     # G = 12, one of the page's Ascend ratios
])
def test_i1_brute_force_shapes(Hq, Hkv, D, P, ctx):
    W = max(-(-c // P) for c in ctx)
    w = _tiny(seed=11 + Hq, ctx=ctx, Hq=Hq, Hkv=Hkv, D=D, P=P, W=W, N=len(ctx) * W + 3)
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert np.max(np.abs(got - _brute_force(w))) <= 1e-12


# ---------------------------------------------------------------------------
# I2: torch's CPU scaled-dot-product attention in FP64 (the textbook routine)
# ---------------------------------------------------------------------------

def _sdpa_reference(w, scale=None):
    import torch.nn.functional as F
    B, Hq, D = w.q.shape
    Hkv = w.k_cache.shape[2]
    P = w.k_cache.shape[1]
    G = Hq // Hkv
    s = float(np.float32(w.scale if scale is None else scale))
    out = torch.zeros(B, Hq, D, dtype=torch.float64)
    for b in range(B):
        n = int(w.context_lens[b])
        if n == 0:
            continue
        npg = -(-n // P)
        idx = w.block_table[b, :npg].long()
        K = w.k_cache.index_select(0, idx).double().reshape(npg * P, Hkv, D)[:n]
        V = w.v_cache.index_select(0, idx).double().reshape(npg * P, Hkv, D)[:n]
        K = K.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()   # [Hq, n, D]
        V = V.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        qb = w.q[b].double().unsqueeze(1)                                   # [Hq, 1, D]
        out[b] = F.scaled_dot_product_attention(qb, K, V, scale=s).squeeze(1)
    return out.numpy()


@pytest.mark.parametrize("B,Hq,Hkv,D,ctx", [
    (4, 40, 8, 128, (1, 127, 129, 300)),
    (3, 16, 2, 256, (256, 1, 385)),
    (2, 24, 2, 256, (5, 130)),
    (2, 8, 8, 64, (33, 200)),
])
def test_i2_matches_torch_sdpa(B, Hq, Hkv, D, ctx):
    w = workloads.build(B, Hq, Hkv, D, ctx, seed=21 + D, max_pages=4, pool="permutation", num_pages=B * 4 + 1)
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert np.max(np.abs(got - _sdpa_reference(w))) <= 1e-12


def test_i2_explicit_scale():
    w = workloads.build(2, 10, 2, 128, (77, 140), seed=3, max_pages=2, pool="packed")
    s = 0.3
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, s)
    assert np.max(np.abs(got - _sdpa_reference(w, scale=s))) <= 1e-12


# ---------------------------------------------------------------------------
# I3: paged layout == contiguous [Hkv, n, D] layout built from the same values
# ---------------------------------------------------------------------------

def test_i3_paged_equals_contiguous():
    w = _tiny(seed=5, ctx=(2, 12, 9, 4), W=3, N=14)
    B, Hq, D = w.q.shape
    _, P, Hkv, _ = w.k_cache.shape
    maxn = int(w.context_lens.max())
    kseq = np.zeros((B, Hkv, maxn, D))
    vseq = np.zeros((B, Hkv, maxn, D))
    kc = _f64(w.k_cache)
    vc = _f64(w.v_cache)
    for b in range(B):
        for t in range(int(w.context_lens[b])):
            page = int(w.block_table[b, t // P])
            kseq[b, :, t, :] = kc[page, t % P]
            vseq[b, :, t, :] = vc[page, t % P]
    paged = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    contig = oracle.contiguous_decode_attention(w.q, kseq, vseq, w.context_lens, w.scale)
    assert np.array_equal(paged, contig)


# ---------------------------------------------------------------------------
# I4: the softmax weights sum to one
# ---------------------------------------------------------------------------

def test_i4_weights_sum_to_one():
    w = _tiny(seed=9)
    _, weights = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table,
                                               w.context_lens, w.scale, return_weights=True)
    assert weights
    for (b, hq), wt in weights.items():
        assert len(wt) == int(w.context_lens[b])
        assert abs(math.fsum(wt.tolist()) - 1.0) <= 1e-14
        assert np.all(wt >= 0)


# ---------------------------------------------------------------------------
# I5: context length 1 returns that V row exactly; I6: uniform scores -> mean
# ---------------------------------------------------------------------------

def test_i5_context_one_returns_v_exactly():
    w = workloads.build(3, 40, 8, 128, (1, 1, 1), seed=13, max_pages=2, pool="permutation", num_pages=8)
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    G = 5
    vc = _f64(w.v_cache)
    for b in range(3):
        page = int(w.block_table[b, 0])
        for hq in range(40):
            assert np.array_equal(got[b, hq], vc[page, 0, hq // G])


def test_i6_uniform_scores_give_mean():
    w = workloads.build(2, 10, 2, 16, (37, 5), seed=17, max_pages=10, pool="packed", page_size=4)
    q0 = torch.zeros_like(w.q)
    got = oracle.paged_decode_attention(q0, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    vc = _f64(w.v_cache)
    for b in range(2):
        n = int(w.context_lens[b])
        rows = [vc[int(w.block_table[b, t // 4]), t % 4] for t in range(n)]
        for hq in range(10):
            h = hq // 5
            mean = np.array([math.fsum(r[h, d] for r in rows) / n for d in range(16)])
            assert np.max(np.abs(got[b, hq] - mean)) <= 1e-12
    # identical keys (q arbitrary) also give equal weights
    k_same = w.k_cache.clone()
    k_same[:] = w.k_cache[0, 0]
    got2 = oracle.paged_decode_attention(w.q, k_same, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert np.max(np.abs(got2 - got)) <= 1e-12


# ---------------------------------------------------------------------------
# Closed form: two tokens with a logit gap of one
# ---------------------------------------------------------------------------

def test_two_token_closed_form():
    # D = 2, one page of 2 slots; q = (1, 0), k0 = (0, 0), k1 = (2, 0), scale 1/2
    # -> logits (0, 1) -> weights (1/(1+e), e/(1+e)); V = identity rows.
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[0.0, 0.0]], [[2.0, 0.0]]]])
    v = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    out = oracle.paged_decode_attention(q, k, v, np.array([[0]]), np.array([2]), 0.5)
    e = math.e
    assert abs(out[0, 0, 0] - 1.0 / (1.0 + e)) <= 1e-15
    assert abs(out[0, 0, 1] - e / (1.0 + e)) <= 1e-15


# ---------------------------------------------------------------------------
# I7: one dominant key placed in the first, a middle and the last partial page
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tstar", [0, 300, 644])
def test_i7_one_hot_limit(tstar):
    n = 645                          # pages 0..5 of 128, the last one partial
    w = workloads.build(1, 5, 1, 128, (n,), seed=23, max_pages=6, pool="permutation", num_pages=9)
    k = w.k_cache.clone()
    q = w.q[0, 0].float()
    page = int(w.block_table[0, tstar // 128])
    # key t* = c * q gives logit c*|q|^2*scale; gap >> ln(n) to the rest
    k[page, tstar % 128, 0] = (q * 8.0).to(torch.bfloat16)
    kt = _f64(k[page, tstar % 128, 0])
    qv = _f64(w.q[0])
    scale = float(np.float32(w.scale))
    got = oracle.paged_decode_attention(w.q, k, w.v_cache, w.block_table, w.context_lens, w.scale)
    # bound: out - v* = sum_{t != t*} w_t (v_t - v*), sum_{t!=t*} w_t <= n e^{-gap}
    kc = _f64(k)
    others = [kc[int(w.block_table[0, t // 128]), t % 128, 0] for t in range(n) if t != tstar]
    vrow = _f64(w.v_cache[page, tstar % 128, 0])
    vmax = float(np.abs(_f64(w.v_cache)).max())
    for hq in range(5):
        top = scale * float(qv[hq] @ kt)
        rest = max(scale * float(qv[hq] @ o) for o in others)
        gap = top - rest
        if hq == 0:
            assert gap > 40.0
        if gap > 40.0:
            bound = (n - 1) * math.exp(-gap) * 2 * vmax + 1e-15
            assert np.max(np.abs(got[0, hq] - vrow)) <= bound


# ---------------------------------------------------------------------------
# I8: permuting the physical page pool changes nothing, bit for bit
# ---------------------------------------------------------------------------

def test_i8_pool_permutation_bit_identical():
    w = _tiny(seed=31, ctx=(11, 3, 8), W=3, N=12)
    N = w.k_cache.shape[0]
    pi = torch.randperm(N, generator=torch.Generator().manual_seed(99))
    k2 = torch.empty_like(w.k_cache)
    v2 = torch.empty_like(w.v_cache)
    k2[pi] = w.k_cache
    v2[pi] = w.v_cache
    bt2 = w.block_table.clone()
    valid = bt2 >= 0
    bt2[valid] = pi[bt2[valid].long()].to(torch.int32)
    a = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    b = oracle.paged_decode_attention(w.q, k2, v2, bt2, w.context_lens, w.scale)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# I9: the [K, V] / [q, 0] embedding identity (orcarouter page, QSA adapter)
# ---------------------------------------------------------------------------

def test_i9_kv_embedding_identity():
    D = 8
    w = _tiny(seed=41, ctx=(6, 11, 1), D=D, W=3, N=10, poison=False)
    kv = torch.cat([w.k_cache, w.v_cache], dim=-1)            # C = [K | V]
    q2 = torch.cat([w.q, torch.zeros_like(w.q)], dim=-1)      # Q' = [Q | 0]
    s = float(np.float32(1.0 / math.sqrt(D)))                 # keep the D-wide scale
    wide = oracle.paged_decode_attention(q2, kv, kv, w.block_table, w.context_lens, s)
    pv = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, s)
    pk = oracle.paged_decode_attention(w.q, w.k_cache, w.k_cache, w.block_table, w.context_lens, s)
    assert np.max(np.abs(wide[..., D:] - pv)) <= 1e-12
    assert np.max(np.abs(wide[..., :D] - pk)) <= 1e-12


# ---------------------------------------------------------------------------
# I10: LSE merge of partials over any partition equals the unsplit result
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cuts", [(0, 700), (0, 128, 256, 700), (0, 1, 2, 699, 700), (0, 0, 350, 350, 700)])
def test_i10_split_merge_partition(cuts):
    rng = np.random.default_rng(5)
    n, D = 700, 32
    qv = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    s = 0.17
    whole = oracle.attend(qv, K, V, s)
    parts = [oracle.partial_attention(qv, K[a:b], V[a:b], s) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.max(np.abs(oracle.lse_merge(parts) - whole)) <= 1e-13


def test_i10_all_empty_is_zero():
    parts = [oracle.partial_attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)] * 3
    assert np.array_equal(oracle.lse_merge(parts), np.zeros(4))


# ---------------------------------------------------------------------------
# I11: the GQA mapping (query heads 5h..5h+4 share KV head h)
# ---------------------------------------------------------------------------

def test_i11_gqa_mapping():
    w = workloads.build(2, 40, 8, 16, (9, 130), seed=51, max_pages=2, pool="permutation", num_pages=5)
    v = torch.empty_like(w.v_cache)
    for h in range(8):
        v[:, :, h, :] = float(h)
    got = oracle.paged_decode_attention(w.q, w.k_cache, v, w.block_table, w.context_lens, w.scale)
    for hq in range(40):
        assert np.max(np.abs(got[:, hq, :] - hq // 5)) <= 1e-13


# ---------------------------------------------------------------------------
# I12: sequences sharing physical pages give identical outputs
# ---------------------------------------------------------------------------

def test_i12_shared_pages():
    w = _tiny(seed=61, ctx=(11, 11, 4), W=3, N=10)
    bt = w.block_table.clone()
    bt[1] = bt[0]
    q = w.q.clone()
    q[1] = q[0]
    got = oracle.paged_decode_attention(q, w.k_cache, w.v_cache, bt, w.context_lens, w.scale)
    assert np.array_equal(got[0], got[1])


# ---------------------------------------------------------------------------
# Special cases: empty context -> exact zeros; NaN in unread slots is ignored
# ---------------------------------------------------------------------------

def test_empty_context_exact_zero_and_poison_ignored():
    w = _tiny(seed=71, ctx=(0, 5, 0, 3))
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    assert np.array_equal(got[2], np.zeros_like(got[2]))
    assert np.all(np.isfinite(got))
    assert torch.isnan(w.k_cache.float()).any()   # the poison really is there


# ---------------------------------------------------------------------------
# Workload recipe checks against the constants the pages print
# ---------------------------------------------------------------------------

def test_workloads_match_page_constants():
    with open(GOLDEN) as f:
        g = json.load(f)
    qw = g["qwen3_14b"]
    for i in (1, 2, 3, 4):
        s = workloads.CONFIG_SHAPES[i]
        assert (s["Hq"], s["Hkv"], s["D"]) == (qw["num_q_heads"], qw["num_kv_heads"], qw["head_dim"])
    assert workloads.PAGE_SIZE == qw["page_size"]
    assert workloads.MAX_CONTEXT == qw["max_context"]
    assert workloads.CONFIG3_LAYERS == qw["num_layers"]
    s5 = workloads.CONFIG_SHAPES[5]
    assert [s5["Hq"], s5["Hkv"]] in g["ascend_local_head_shapes_d256"]["pairs"]
    assert s5["D"] == g["ascend_local_head_shapes_d256"]["head_dim"]


def test_config1_recipe():
    w = workloads.config(1)
    assert w.context_lens.tolist() == [1, 130]
    assert sorted(w.block_table.flatten().tolist()) == [0, 1, 2, 3]
    assert w.q.dtype == torch.bfloat16 and tuple(w.k_cache.shape) == (4, 128, 8, 128)
    assert w.scale == float(np.float32(1 / math.sqrt(128)))


def test_config4_recipe():
    w = workloads.config(4)
    ctx = w.context_lens
    assert int(ctx.min()) >= 1 and int(ctx.max()) <= 4096
    npages = [-(-int(c) // 128) for c in ctx]
    assert w.k_cache.shape[0] == sum(npages)
    used = torch.cat([w.block_table[b, :n] for b, n in enumerate(npages)])
    assert sorted(used.tolist()) == list(range(sum(npages)))      # each page used once
    for b, n in enumerate(npages):
        assert (w.block_table[b, n:] == -1).all()


# ---------------------------------------------------------------------------
# Mutation checks: a planted mistake in the oracle fails the pins above
# ---------------------------------------------------------------------------

def _planted(monkeypatch, kind):
    real_attend = oracle_decode.attend
    real_gather = oracle_decode.gather_sequence
    if kind == "drop_scale":
        monkeypatch.setattr(oracle_decode, "attend",
                            lambda qv, K, V, s, rw=False: real_attend(qv, K, V, 1.0, rw))
    elif kind == "transpose_kv":
        monkeypatch.setattr(oracle_decode, "attend",
                            lambda qv, K, V, s, rw=False: real_attend(qv, V, K, s, rw))
    elif kind == "drop_last_token":
        monkeypatch.setattr(oracle_decode, "attend",
                            lambda qv, K, V, s, rw=False: real_attend(qv, K[:max(1, len(K) - 1)], V[:max(1, len(V) - 1)], s, rw))
    elif kind == "wrong_slot":
        def bad_gather(cache, row, n):
            g = real_gather(cache, row, n + 1 if n % cache.shape[1] else n)
            return g[-n:]
        monkeypatch.setattr(oracle_decode, "gather_sequence", bad_gather)
    elif kind == "sign":
        monkeypatch.setattr(oracle_decode, "attend",
                            lambda qv, K, V, s, rw=False: real_attend(qv, K, V, -s, rw))


@pytest.mark.parametrize("kind", ["drop_scale", "transpose_kv", "drop_last_token", "wrong_slot", "sign"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    w = _tiny(seed=81, ctx=(1, 4, 5, 11), poison=False)
    ref = _brute_force(w)
    _planted(monkeypatch, kind)
    got = oracle.paged_decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert not (np.max(np.abs(got - ref)) <= 1e-12)


def test_planted_head_mapping_is_caught(monkeypatch):
    # a modulo head mapping (hq % Hkv) instead of consecutive grouping
    w = workloads.build(1, 10, 2, 8, (6,), seed=91, max_pages=1, pool="permutation", num_pages=2, page_size=8)
    ref = _sdpa_reference(w)
    q_perm = w.q.clone()
    order = [(hq % 2) * 5 + hq // 2 for hq in range(10)]   # mapping hq -> hq % 2 via a relabel
    got = oracle.paged_decode_attention(q_perm[:, order], w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert not (np.max(np.abs(got - ref)) <= 1e-12)
