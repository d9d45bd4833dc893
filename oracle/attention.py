"""fp64 decode attention over contiguous K/V — the oracle's definition (test infrastructure).

"PagedAttention: Optimizing KV Cache in vLLM" (grasp.study lesson), §3 "Making it
Work: The PagedAttention Kernel": the paged kernel follows the block table, walks the
blocks in logical order and keeps a running softmax normalisation, and its result is
the same as attention over a contiguous layout; paging is a layout change only.  So
this module writes out plain softmax attention for one query token per sequence, on
each sequence's logical (contiguous) K and V, in float64:

    x_t   = scale * <q[s, h], K_s[t, g]>                   for t < L_s
    out   = sum_t exp(x_t - max x) V_s[t, g] / sum_t exp(x_t - max x)

with query head h reading KV head g = h // G (G = Hq / Hkv, contiguous groups; the
"PagedAttention" kongchang page lists grouped-query attention among KV-cache
optimisations, and G = 1 is ordinary multi-head attention).  A sequence with
L_s = 0 has no keys; its output is defined as zero.

Decoding the stored K/V to float64 uses ``codecs``: bf16 and e4m3fn are exact in
float64, and the fp8 dequantisation code * scale is an exact float64 product.

Pinned by ``tests/test_oracle_attention.py``: a scalar brute force with math.fsum,
a hand-worked fixture (tests/golden/attention_hand_example.json), closed forms
(L = 1, q = 0, L = 2), torch's float64 scaled_dot_product_attention and the
shift / affine / permutation invariants of softmax attention.
"""
from __future__ import annotations

import numpy as np

from . import codecs


def q_to_f64(q: np.ndarray, q_dtype: str) -> np.ndarray:
    if q_dtype == "f32":
        return np.asarray(q, dtype=np.float32).astype(np.float64)
    if q_dtype == "bf16":
        return codecs.bf16_to_f64(q)
    raise ValueError(q_dtype)


def kv_to_f64(x: np.ndarray, kv_dtype: str, scale=1.0) -> np.ndarray:
    """Stored K or V values -> float64 as the cache holds them.

    f32 / bf16 are stored as given.  For e4m3fn the input holds the bf16 values that
    were written; the cache holds their quantised codes, dequantised as code * scale.
    """
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return codecs.bf16_to_f64(x)
    if kv_dtype == "fp8_e4m3fn":
        codes = codecs.quantize_bf16_to_e4m3fn(x, codecs.inverse_scale(scale))
        return codecs.e4m3fn_to_f64(codes) * np.float64(np.float32(scale))
    raise ValueError(kv_dtype)


def decode_attention(q: np.ndarray, ks, vs, scale: float, group_size: int) -> np.ndarray:
    """Softmax attention of one query token per sequence over contiguous K/V, in float64.

    q:  [B, Hq, D] float64.
    ks, vs: sequences of [L_s, Hkv, D] float64 arrays (logical token order).
    Returns [B, Hq, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = int(group_size)
    assert Hq % G == 0
    Hkv = Hq // G
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        K = np.asarray(ks[s], dtype=np.float64)
        V = np.asarray(vs[s], dtype=np.float64)
        if K.shape[0] == 0:
            continue
        assert K.shape[1:] == (Hkv, D) and V.shape == K.shape
        for g in range(Hkv):
            Qg = q[s, g * G:(g + 1) * G]                 # [G, D]
            X = scale * (Qg @ K[:, g, :].T)               # [G, L]
            W = np.exp(X - X.max(axis=1, keepdims=True))  # [G, L]
            out[s, g * G:(g + 1) * G] = (W @ V[:, g, :]) / W.sum(axis=1, keepdims=True)
    return out


def decode_case(case, seqs=None) -> np.ndarray:
    """Oracle output for a ``synth.DecodeCase`` (optionally only the listed sequences).

    Returns [len(seqs), Hq, D] float64 in the order of ``seqs``.
    """
    wl = case.wl
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    q = q_to_f64(case.q[seqs], wl.q_dtype)
    ks = [kv_to_f64(case.seq_k(s), wl.kv_dtype, case.k_scale) for s in seqs]
    vs = [kv_to_f64(case.seq_v(s), wl.kv_dtype, case.v_scale) for s in seqs]
    return decode_attention(q, ks, vs, case.scale, wl.group_size)


def prefix_step_case(case, seqs=None) -> np.ndarray:
    """Oracle output for a ``synth.PrefixStepCase`` after its one-token append step."""
    wl = case.wl
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    q = q_to_f64(case.q[seqs], wl.q_dtype)
    ks, vs = [], []
    for i in seqs:
        k, v = case.logical_kv(i)
        ks.append(kv_to_f64(k, wl.kv_dtype))
        vs.append(kv_to_f64(v, wl.kv_dtype))
    return decode_attention(q, ks, vs, case.scale, wl.group_size)
