"""Pins for the fp64 causal multi-query oracle (CPU only).

``oracle.attention.prefill_attention`` is tied to: hand-worked values
(tests/golden/prefill_hand_example.json), a scalar brute force with math.fsum, the decode
oracle when every sequence has one query, torch's float64 scaled_dot_product_attention
with a bottom-right causal mask built by torch.tril, closed forms, and the property that
splitting a sequence's queries into chunks does not change any output.  Broken copies
(top-left mask alignment, a strict mask, a wrong head map, a missing scale) must fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_hand_example.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _case_arrays(case):
    q = np.array(case["q"], dtype=np.float64)
    ks = [np.array(k, dtype=np.float64) for k in case["k"]]
    vs = [np.array(v, dtype=np.float64) for v in case["v"]]
    return q, ks, vs, case["q_lens"], case["scale"], q.shape[1] // case["num_kv_heads"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    q, ks, vs, n, scale, G = _case_arrays(case)
    got = oatt.prefill_attention(q, ks, vs, n, scale, G)
    assert np.allclose(got, np.array(case["expected"]), rtol=0, atol=1e-12)


def _brute(q, ks, vs, q_lens, scale, G):
    """Scalar loops over positions with math.exp / math.fsum."""
    T, Hq, D = q.shape
    out = np.zeros_like(q)
    row = 0
    for s, n in enumerate(q_lens):
        L = ks[s].shape[0]
        for i in range(n):
            P = L - n + i
            for h in range(Hq):
                if P < 0:
                    continue
                g = h // G
                x = [scale * math.fsum(q[row + i, h, d] * ks[s][t, g, d] for d in range(D))
                     for t in range(P + 1)]
                mx = max(x)
                w = [math.exp(v - mx) for v in x]
                den = math.fsum(w)
                for d in range(D):
                    out[row + i, h, d] = math.fsum(w[t] * vs[s][t, g, d] for t in range(P + 1)) / den
        row += n
    return out


def _rand(rng, lens, q_lens, Hkv, G, D):
    q = rng.standard_normal((sum(q_lens), Hkv * G, D))
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    return q, ks, vs


@pytest.mark.parametrize("G", [1, 2, 3])
def test_brute_force_tiny(G):
    rng = np.random.default_rng(20 + G)
    lens, q_lens = [1, 4, 5, 3, 2], [1, 4, 2, 3, 3]     # n = L, n < L and n > L
    q, ks, vs = _rand(rng, lens, q_lens, 2, G, 3)
    got = oatt.prefill_attention(q, ks, vs, q_lens, 0.8, G)
    assert np.max(np.abs(got - _brute(q, ks, vs, q_lens, 0.8, G))) < 1e-13


def test_one_query_per_sequence_is_decode():
    rng = np.random.default_rng(30)
    lens = [1, 7, 40, 129]
    q, ks, vs = _rand(rng, lens, [1] * 4, 2, 4, 16)
    got = oatt.prefill_attention(q, ks, vs, [1] * 4, 0.25, 4)
    ref = oatt.decode_attention(q, ks, vs, 0.25, 4)
    assert np.max(np.abs(got - ref)) < 1e-13


@pytest.mark.parametrize("G,lens,q_lens", [(1, [17, 40], [17, 40]), (4, [64, 129, 33], [16, 5, 33]),
                                           (8, [250, 3], [100, 1])])
def test_against_torch_sdpa_with_bottom_right_mask(G, lens, q_lens):
    rng = np.random.default_rng(40 + G)
    Hkv, D = 2, 16
    q, ks, vs = _rand(rng, lens, q_lens, Hkv, G, D)
    scale = 1 / math.sqrt(D)
    got = oatt.prefill_attention(q, ks, vs, q_lens, scale, G)
    row = 0
    for s, (L, n) in enumerate(zip(lens, q_lens)):
        Q = torch.from_numpy(q[row:row + n]).permute(1, 0, 2).unsqueeze(0).contiguous()   # [1, Hq, n, D]
        K = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        V = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        assert np.max(np.abs(got[row:row + n] - ref[0].permute(1, 0, 2).numpy())) < 1e-12
        row += n


def test_first_prefill_query_returns_the_first_value_exactly():
    rng = np.random.default_rng(50)
    lens = [9, 30]
    q, ks, vs = _rand(rng, lens, lens, 2, 2, 8)
    got = oatt.prefill_attention(q, ks, vs, lens, 0.3, 2)
    for s, row in enumerate([0, 9]):
        for h in range(4):
            assert np.array_equal(got[row, h], vs[s][0, h // 2])


def test_zero_queries_give_prefix_means():
    rng = np.random.default_rng(51)
    L = 12
    _, ks, vs = _rand(rng, [L], [L], 1, 1, 5)
    got = oatt.prefill_attention(np.zeros((L, 1, 5)), ks, vs, [L], 1.0, 1)
    for P in range(L):
        assert np.allclose(got[P, 0], vs[0][:P + 1, 0].mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("split", [1, 7, 20])
def test_chunking_the_queries_changes_nothing(split):
    """Queries of one sequence computed in two chunks (the first over the tokens that exist
    when it runs) equal the queries computed together."""
    rng = np.random.default_rng(60 + split)
    L, n = 50, 32
    q, ks, vs = _rand(rng, [L], [n], 2, 2, 8)
    whole = oatt.prefill_attention(q, ks, vs, [n], 0.4, 2)
    L1 = L - (n - split)
    first = oatt.prefill_attention(q[:split], [ks[0][:L1]], [vs[0][:L1]], [split], 0.4, 2)
    second = oatt.prefill_attention(q[split:], ks, vs, [n - split], 0.4, 2)
    assert np.allclose(whole[:split], first, atol=1e-14)
    assert np.allclose(whole[split:], second, atol=1e-14)


def test_queries_past_the_context_are_zero():
    rng = np.random.default_rng(70)
    q, ks, vs = _rand(rng, [3], [5], 1, 2, 4)
    got = oatt.prefill_attention(q, ks, vs, [5], 0.5, 2)
    assert np.all(got[:2] == 0) and np.all(np.isfinite(got[2:]))


# ---- planted mistakes: broken copies of the oracle must fail the pins ------------------

def _broken_top_left(q, ks, vs, q_lens, scale, G):
    # Query i attends to tokens 0..i whatever the context length.
    outs, row = [], 0
    for s, n in enumerate(q_lens):
        m = min(n, ks[s].shape[0])
        outs.append(oatt.prefill_attention(q[row:row + n], [ks[s][:n]], [vs[s][:n]], [n], scale, G)
                    if m == n else oatt.prefill_attention(q[row:row + n], [ks[s]], [vs[s]], [n], scale, G))
        row += n
    return np.concatenate(outs)


def _broken_strict_mask(q, ks, vs, q_lens, scale, G):
    # The query does not see its own token.
    out = np.zeros_like(q)
    row = 0
    for s, n in enumerate(q_lens):
        L = ks[s].shape[0]
        for i in range(n):
            P = L - n + i
            if P >= 1:
                out[row + i:row + i + 1] = oatt.decode_attention(q[row + i:row + i + 1], [ks[s][:P]],
                                                                 [vs[s][:P]], scale, G)
        row += n
    return out


def _broken_head_map(q, ks, vs, q_lens, scale, G):
    T, Hq, D = q.shape
    Hkv = Hq // G
    perm = [(h % Hkv) * G + (h // Hkv) for h in range(Hq)]
    inv = np.argsort(perm)
    return oatt.prefill_attention(q[:, inv], ks, vs, q_lens, scale, G)[:, perm]


def _broken_no_scale(q, ks, vs, q_lens, scale, G):
    return oatt.prefill_attention(q, ks, vs, q_lens, 1.0, G)


@pytest.mark.parametrize("broken", [_broken_top_left, _broken_strict_mask, _broken_head_map,
                                    _broken_no_scale])
def test_pins_reject_planted_mistakes(broken):
    caught = False
    for case in _golden_cases():
        q, ks, vs, n, scale, G = _case_arrays(case)
        got = broken(q, ks, vs, n, scale, G)
        caught |= not np.allclose(got, np.array(case["expected"]), atol=1e-12)
    rng = np.random.default_rng(80)
    lens, q_lens = [6, 5], [3, 5]
    q, ks, vs = _rand(rng, lens, q_lens, 2, 2, 3)
    caught_rand = not np.allclose(broken(q, ks, vs, q_lens, 0.7, 2), _brute(q, ks, vs, q_lens, 0.7, 2),
                                  atol=1e-9)
    assert caught or caught_rand


@pytest.mark.parametrize("name", ["prefill_tiny_fp32", "prefill_llama3_8b_bf16", "prefill_fp8_kv",
                                  "chunked_prefill_llama3_8b_bf16", "spec_verify_llama3_8b_bf16"])
def test_prefill_case_matches_sdpa_on_synthetic_workloads(name):
    """The case plumbing (row -> sequence and position, dtype decode, fp8 dequant) against
    torch SDPA with a bottom-right causal mask, on a scaled-down draw of each workload."""
    from synth import WORKLOADS, make_prefill_case
    from oracle import codecs

    wl = WORKLOADS[name]
    wl = wl.scaled(batch=3, length_dist=("uniform", 1, 70),
                   query_dist=wl.query_dist if wl.query_dist[0] != "fixed" else ("fixed", 9))
    case = make_prefill_case(wl, seed=4)
    rows = list(range(case.num_q_tokens))
    got = oatt.prefill_case(case, rows)
    G, D = wl.group_size, wl.head_dim

    def dec(x, sc):
        if wl.kv_dtype == "f32":
            return torch.from_numpy(x.astype(np.float64))
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        if wl.kv_dtype == "bf16":
            return t.double()
        inv = codecs.inverse_scale(sc)
        return (t.float() * float(inv)).clamp(-448, 448).to(torch.float8_e4m3fn).double() * float(np.float32(sc))

    for s in range(wl.batch):
        a, b = int(case.query_start[s]), int(case.query_start[s + 1])
        n, L = b - a, int(case.lengths[s])
        if wl.q_dtype == "f32":
            q = torch.from_numpy(case.q[a:b].astype(np.float64))
        else:
            q = torch.from_numpy(case.q[a:b].view(np.int16)).view(torch.bfloat16).double()
        K = dec(case.seq_k(s), case.k_scale).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        V = dec(case.seq_v(s), case.v_scale).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(q.permute(1, 0, 2).unsqueeze(0).contiguous(),
                                                               K, V, attn_mask=mask, scale=case.scale)
        assert np.max(np.abs(got[a:b] - ref[0].permute(1, 0, 2).numpy())) < 1e-11
