"""FP64 CPU oracle for the attention prologue: QK-norm, NeoX RoPE, KV write.

TEST INFRASTRUCTURE ONLY (as the rest of this package): nothing on the product
path imports it, and it shares no code with the HIP library.

What it computes, and where the pages define it
------------------------------------------------
"Qwen 3" (TensorSharp docs), section 3 "Forward graph": after the QKV
projection, every query head and every key head goes through its own RMSNorm
(weights attn_q_norm / attn_k_norm, one value per head dim), then NeoX-style
RoPE at the token's position, then K and V are appended to the cache. Section
4.1 "Attention": QK-norm is a per-head RMSNorm with head_dim-sized weights;
RoPE is NeoX-style with frequencies precomputed from the RoPE base and scale.
Section 4.3 "Normalization": epsilon comes from the config (typically 1e-6).
Section 5 "Parameters": the base (about 1e6 for Qwen 3) and a frequency scale
divisor. "Qwen3-14B" (pypto-lib models page), section "decode_fwd": the decode
layer runs Q/K norm -> RoPE -> KV cache write in front of paged attention, the
attention kernel's phase 0.

For a head vector x of D values, with weight w, position p:

    y_d        = x_d / sqrt(mean(x^2) + eps) * w_d                   (RMSNorm)
    theta_i    = p * base^(-2i/D) / scale,            i = 0 .. D/2-1
    out_i      = y_i cos(theta_i) - y_{i+D/2} sin(theta_i)          (NeoX halves)
    out_{i+D/2} = y_{i+D/2} cos(theta_i) + y_i sin(theta_i)

Readings of points the pages leave open
---------------------------------------
P1  NeoX style pairs dim i with dim i + D/2 (the two halves), not adjacent
    dims; the rotation is by +theta (out = (y_i + j y_{i+D/2}) e^{j theta}).
P2  The frequency scale divides the frequency: theta_i = p * base^(-2i/D) / scale.
P3  RMSNorm divides by sqrt(mean of squares + eps), then multiplies by w.
P4  The prologue's q output is not yet multiplied by 1/sqrt(head_dim): the
    attention call applies its ``scale``, as the pages' order (norm, RoPE, then
    the 1/sqrt(head_dim) factor, then attention) allows.
P5  V is neither normalised nor rotated; it is written to the cache as given.
    K is written after norm and RoPE. A negative slot marks a padding token:
    its q is still computed, nothing is written to the cache (as paged_kv_write).

All arithmetic is FP64; inputs are BF16 values widened exactly.
"""

from __future__ import annotations

import numpy as np

from .decode import paged_kv_write, paged_kv_write_fp8

__all__ = ["rms_norm_heads", "rope_neox", "rope_angles", "attention_prologue"]


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rms_norm_heads(x, w, eps):
    """Per-head RMSNorm over the last axis ("Qwen 3" section 4.1, QK-norm)."""
    x = _f64(x)
    w = _f64(w)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(np.float32(eps))) * w


def rope_angles(positions, head_dim, base, scale):
    """theta[t, i] = positions[t] * base^(-2i/D) / scale, i < D/2 (reading P2)."""
    pos = _f64(positions).reshape(-1, 1)
    i = np.arange(head_dim // 2, dtype=np.float64).reshape(1, -1)
    inv_freq = np.power(float(np.float32(base)), -2.0 * i / head_dim) / float(np.float32(scale))
    return pos * inv_freq


def rope_neox(x, positions, base, scale):
    """NeoX RoPE over the last axis of x [T, H, D] at positions [T] (reading P1)."""
    x = _f64(x)
    D = x.shape[-1]
    h = D // 2
    th = rope_angles(positions, D, base, scale)[:, None, :]  # [T, 1, D/2]
    c, s = np.cos(th), np.sin(th)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention_prologue(q, k, v, q_norm_w, k_norm_w, positions, slot_mapping, eps,
                       rope_base, rope_scale, k_cache, v_cache):
    """QK-norm, NeoX RoPE and the KV write of T new tokens.

    q [T, Hq, D], k and v [T, Hkv, D] (the QKV projection's outputs), weights
    [D], positions and slot_mapping [T]. Returns (q_out FP64 [T, Hq, D],
    k_cache FP64, v_cache FP64): the caches are copies with the rows of every
    non-padding token written (K after norm and RoPE, V as given).
    """
    q_out = rope_neox(rms_norm_heads(q, q_norm_w, eps), positions, rope_base, rope_scale)
    k_rot = rope_neox(rms_norm_heads(k, k_norm_w, eps), positions, rope_base, rope_scale)
    kc, vc = paged_kv_write(_f64(k_cache), _f64(v_cache), k_rot, _f64(v), slot_mapping)
    return q_out, kc, vc


def round_bf16(x) -> np.ndarray:
    """FP64 values rounded once to the nearest BF16 value (8 significant bits;
    ties to even; spacing 2^-133 below 2^-126), returned as FP64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| = m * 2^e with 0.5 <= m < 1
    step = np.maximum(e - 8, -133)          # exponent of the BF16 spacing at x
    return np.ldexp(np.rint(np.ldexp(x, -step)), step)


def attention_prologue_fp8(q, k, v, q_norm_w, k_norm_w, positions, slot_mapping, eps,
                           rope_base, rope_scale, k_scale, v_scale, k_codes, v_codes):
    """The prologue writing FP8-E4M3 pools: the K rows of ``attention_prologue``
    rounded to BF16 (the row the BF16 pools would hold), then stored as
    ``paged_kv_write_fp8`` stores a BF16 row (codes of x / k_scale); V as
    given, codes of v / v_scale. Reading: the pages name the fp8_e4m3 cache
    but not where the rounding happens; quantising the BF16 row makes the FP8
    prologue the BF16 prologue followed by the FP8 write. Returns (q_out FP64,
    k_codes, v_codes) with the codes as new uint8 arrays."""
    q_out = rope_neox(rms_norm_heads(q, q_norm_w, eps), positions, rope_base, rope_scale)
    k_rot = round_bf16(rope_neox(rms_norm_heads(k, k_norm_w, eps), positions, rope_base,
                                  rope_scale))
    kc, vc = paged_kv_write_fp8(k_codes, v_codes, k_rot, _f64(v), k_scale, v_scale, slot_mapping)
    return q_out, kc, vc
