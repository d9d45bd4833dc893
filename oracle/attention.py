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

Several query tokens per sequence (``prefill_attention``): "What is PagedAttention?"
(qubittool glossary), "How It Works: Map Logical to Physical Blocks", has a prefill
allocate blocks for the whole input, and "PagedAttention: Optimizing KV Cache in vLLM"
(grasp.study), "Conclusion", points at speculative decoding, where a target model checks
several drafted tokens at once.  Neither page writes out the attention of those query
tokens; the plainest reading, and the one decode already follows (the new token attends
to every cached token and to itself), is causal attention: the sequence's last n_s tokens
are the queries, and the query at position P attends to tokens 0..P.  A prefill is
n_s = L_s, a prefill chunk or a verification is n_s < L_s, and n_s = 1 is decode.
Pinned by ``tests/test_oracle_prefill.py``.
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
        codes = codecs.bf16_to_e4m3fn_table(codecs.inverse_scale(scale))[np.asarray(x, dtype=np.uint16)]
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


def causal_query(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, P: int, scale: float,
                 group_size: int) -> np.ndarray:
    """One query token at position P over tokens 0..P of K / V ([L, Hkv, D] float64).

    q_row: [Hq, D] float64.  Returns [Hq, D]; zero when P < 0.
    """
    Hq, D = q_row.shape
    G = int(group_size)
    out = np.zeros((Hq, D), dtype=np.float64)
    if P < 0:
        return out
    Kp, Vp = K[:P + 1], V[:P + 1]
    for g in range(Hq // G):
        Qg = q_row[g * G:(g + 1) * G]                    # [G, D]
        X = scale * (Qg @ Kp[:, g, :].T)                  # [G, P+1]
        W = np.exp(X - X.max(axis=1, keepdims=True))
        out[g * G:(g + 1) * G] = (W @ Vp[:, g, :]) / W.sum(axis=1, keepdims=True)
    return out


def prefill_attention(q: np.ndarray, ks, vs, q_lens, scale: float, group_size: int) -> np.ndarray:
    """Causal softmax attention of the last n_s tokens of every sequence, in float64.

    q:       [sum n_s, Hq, D] float64; sequence s's queries are rows
             sum(n_0..n_{s-1}) .. + n_s, in position order.
    ks, vs:  sequences of [L_s, Hkv, D] float64 arrays (logical token order), holding every
             token of the sequence, the queries' own tokens included.
    q_lens:  n_s per sequence.  Query i of sequence s sits at position P = L_s - n_s + i and
             attends to tokens 0..P; a query with P < 0 (n_s > L_s) attends to nothing and
             its output is zero.
    Returns [sum n_s, Hq, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    G = int(group_size)
    assert Hq % G == 0
    q_lens = [int(n) for n in q_lens]
    assert sum(q_lens) == T
    out = np.zeros((T, Hq, D), dtype=np.float64)
    row = 0
    for s, n in enumerate(q_lens):
        K = np.asarray(ks[s], dtype=np.float64)
        V = np.asarray(vs[s], dtype=np.float64)
        L = K.shape[0]
        assert V.shape == K.shape and (L == 0 or K.shape[1:] == (Hq // G, D))
        for i in range(n):
            out[row + i] = causal_query(q[row + i], K, V, L - n + i, scale, G)
        row += n
    return out


def prefill_case(case, rows=None) -> np.ndarray:
    """Oracle output for a ``synth.PrefillCase``, for all query rows or the listed ones.

    Returns [len(rows), Hq, D] float64 in the order of ``rows`` (global query-row indices).
    """
    wl = case.wl
    qs = np.asarray(case.query_start, dtype=np.int64)
    rows = list(range(int(qs[-1]))) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(rows), wl.num_q_heads, wl.head_dim), dtype=np.float64)
    decoded = {}
    for k, r in enumerate(rows):
        s = int(np.searchsorted(qs, r, side="right") - 1)
        if s not in decoded:
            decoded[s] = (kv_to_f64(case.seq_k(s), wl.kv_dtype, case.k_scale),
                          kv_to_f64(case.seq_v(s), wl.kv_dtype, case.v_scale))
        K, V = decoded[s]
        n = int(qs[s + 1] - qs[s])
        P = int(case.lengths[s]) - n + (r - int(qs[s]))
        out[k] = causal_query(q_to_f64(case.q[r], wl.q_dtype), K, V, P, case.scale, wl.group_size)
    return out
