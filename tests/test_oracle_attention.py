"""Pins for the fp64 attention oracle (CPU only).

Each test ties ``oracle.attention`` to something other than itself: a scalar brute
force with math.fsum, hand-worked values, closed forms, torch's float64
scaled_dot_product_attention, and invariants that softmax attention must satisfy.
The "planted mistake" tests run deliberately broken copies of the oracle and check
that these pins reject them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_hand_example.json")


def _brute(q, ks, vs, scale, G):
    """Scalar loops, math.exp and math.fsum: one query row at a time."""
    B, Hq, D = q.shape
    out = np.zeros_like(q)
    for s in range(B):
        L = ks[s].shape[0]
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            x = [scale * math.fsum(q[s, h, d] * ks[s][t, g, d] for d in range(D)) for t in range(L)]
            mx = max(x)
            w = [math.exp(v - mx) for v in x]
            den = math.fsum(w)
            for d in range(D):
                out[s, h, d] = math.fsum(w[t] * vs[s][t, g, d] for t in range(L)) / den
    return out


def _rand_case(rng, B, Hq, Hkv, D, lens):
    q = rng.standard_normal((B, Hq, D))
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    return q, ks, vs


@pytest.mark.parametrize("G", [1, 2, 3])
def test_brute_force_tiny(G):
    rng = np.random.default_rng(7 + G)
    Hkv, D = 2, 3
    lens = [1, 2, 3, 5]
    q, ks, vs = _rand_case(rng, len(lens), Hkv * G, Hkv, D, lens)
    got = oatt.decode_attention(q, ks, vs, 0.7, G)
    ref = _brute(q, ks, vs, 0.7, G)
    assert np.max(np.abs(got - ref)) < 1e-13


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    G = q.shape[1] // case["num_kv_heads"]
    got = oatt.decode_attention(q, [k], [v], case["scale"], G)
    assert np.allclose(got, np.array(case["expected"]), rtol=0, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    q, ks, vs = _rand_case(rng, 3, 4, 2, 8, [1, 1, 1])
    got = oatt.decode_attention(q, ks, vs, 0.3, 2)
    for s in range(3):
        for h in range(4):
            assert np.array_equal(got[s, h], vs[s][0, h // 2])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    _, ks, vs = _rand_case(rng, 2, 2, 2, 5, [7, 33])
    q = np.zeros((2, 2, 5))
    got = oatt.decode_attention(q, ks, vs, 1.0, 1)
    for s in range(2):
        assert np.allclose(got[s], vs[s].mean(axis=0), atol=1e-14)


def test_two_tokens_logistic_closed_form():
    rng = np.random.default_rng(3)
    q, ks, vs = _rand_case(rng, 1, 1, 1, 6, [2])
    scale = 0.4
    delta = scale * q[0, 0] @ (ks[0][0, 0] - ks[0][1, 0])
    sig = 1.0 / (1.0 + math.exp(-delta))
    expect = sig * vs[0][0, 0] + (1 - sig) * vs[0][1, 0]
    got = oatt.decode_attention(q, ks, vs, scale, 1)
    assert np.allclose(got[0, 0], expect, atol=1e-14)


def test_empty_sequence_is_zero():
    rng = np.random.default_rng(4)
    q, ks, vs = _rand_case(rng, 2, 4, 4, 8, [0, 3])
    got = oatt.decode_attention(q, ks, vs, 0.5, 1)
    assert np.all(got[0] == 0)
    assert np.all(np.isfinite(got[1]))


@pytest.mark.parametrize("G,lens", [(1, [1, 17, 40]), (4, [3, 64, 129]), (8, [250, 2, 1])])
def test_against_torch_sdpa_float64(G, lens):
    rng = np.random.default_rng(5 + G)
    Hkv, D = 2, 16
    q, ks, vs = _rand_case(rng, len(lens), Hkv * G, Hkv, D, lens)
    scale = 1 / math.sqrt(D)
    got = oatt.decode_attention(q, ks, vs, scale, G)
    for s, L in enumerate(lens):
        Q = torch.from_numpy(q[s]).reshape(1, Hkv * G, 1, D)
        K = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        V = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        assert np.max(np.abs(got[s] - ref[0, :, 0].numpy())) < 1e-12


def test_key_shift_invariance():
    rng = np.random.default_rng(8)
    q, ks, vs = _rand_case(rng, 2, 4, 2, 8, [9, 30])
    base = oatt.decode_attention(q, ks, vs, 0.35, 2)
    u = rng.standard_normal((1, 2, 8)) * 5
    shifted = oatt.decode_attention(q, [k + u for k in ks], vs, 0.35, 2)
    assert np.allclose(base, shifted, atol=1e-12)


def test_value_affine_equivariance():
    rng = np.random.default_rng(9)
    q, ks, vs = _rand_case(rng, 2, 2, 2, 4, [5, 12])
    base = oatt.decode_attention(q, ks, vs, 0.5, 1)
    a, b = -1.7, rng.standard_normal(4)
    got = oatt.decode_attention(q, ks, [a * v + b for v in vs], 0.5, 1)
    assert np.allclose(got, a * base + b, atol=1e-12)


def test_joint_token_permutation_invariance():
    rng = np.random.default_rng(10)
    q, ks, vs = _rand_case(rng, 1, 4, 1, 8, [37])
    perm = rng.permutation(37)
    base = oatt.decode_attention(q, ks, vs, 0.3, 4)
    got = oatt.decode_attention(q, [ks[0][perm]], [vs[0][perm]], 0.3, 4)
    assert np.allclose(base, got, atol=1e-13)


def test_large_logits_stay_finite():
    rng = np.random.default_rng(11)
    q, ks, vs = _rand_case(rng, 1, 2, 1, 8, [50])
    got = oatt.decode_attention(q * 300.0, ks, vs, 1.0, 2)
    assert np.all(np.isfinite(got))


# ---- planted mistakes: broken copies of the oracle must fail the pins ------------------

def _broken_no_scale(q, ks, vs, scale, G):
    return oatt.decode_attention(q, ks, vs, 1.0, G)


def _broken_head_map(q, ks, vs, scale, G):
    # q head h reads kv head h % Hkv instead of h // G.
    B, Hq, D = q.shape
    Hkv = Hq // G
    perm = [(h % Hkv) * G + (h // Hkv) for h in range(Hq)]
    inv = np.argsort(perm)
    out = oatt.decode_attention(q[:, inv], ks, vs, scale, G)
    return out[:, perm]


def _broken_no_max_shift(q, ks, vs, scale, G):
    out = np.zeros_like(q)
    for s in range(q.shape[0]):
        for h in range(q.shape[1]):
            x = scale * ks[s][:, h // G] @ q[s, h]
            w = np.exp(x)
            out[s, h] = (w @ vs[s][:, h // G]) / max(w.sum(), 1e-300)
    return out


def _broken_transposed_value(q, ks, vs, scale, G):
    return oatt.decode_attention(q, ks, [v[::-1] for v in vs], scale, G)


@pytest.mark.parametrize("broken", [_broken_no_scale, _broken_head_map, _broken_no_max_shift,
                                    _broken_transposed_value])
def test_pins_reject_planted_mistakes(broken):
    caught = False
    for case in _golden_cases():
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        G = q.shape[1] // case["num_kv_heads"]
        with np.errstate(over="ignore", invalid="ignore"):
            got = broken(q, [k], [v], case["scale"], G)
        if not np.allclose(got, np.array(case["expected"]), atol=1e-12):
            caught = True
    if not caught:
        # Large logits catch a missing max shift (exp overflows); a brute force catches the rest.
        rng = np.random.default_rng(12)
        q, ks, vs = _rand_case(rng, 2, 4, 2, 3, [3, 4])
        q = q * 400
        with np.errstate(over="ignore", invalid="ignore"):
            got = broken(q, ks, vs, 0.9, 2)
        caught = not np.allclose(got, _brute(q, ks, vs, 0.9, 2), atol=1e-9)
    assert caught


@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b_bf16", "fp8_kv", "long_ctx_splitk_bf16"])
def test_decode_case_matches_sdpa_on_synthetic_workloads(name):
    """The case plumbing (dtype decode, fp8 dequant, head grouping) against torch SDPA."""
    from synth import WORKLOADS, make_decode_case
    from oracle import codecs

    wl = WORKLOADS[name].scaled(batch=3, length_dist=("uniform", 1, 70))
    case = make_decode_case(wl, seed=3)
    got = oatt.decode_case(case)
    G, D = wl.group_size, wl.head_dim
    for s in range(wl.batch):
        if wl.q_dtype == "f32":
            q = torch.from_numpy(case.q[s].astype(np.float64))
        else:
            q = torch.from_numpy(case.q[s].view(np.int16)).view(torch.bfloat16).double()
        def dec(x, sc):
            if wl.kv_dtype == "f32":
                return torch.from_numpy(x.astype(np.float64))
            t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
            if wl.kv_dtype == "bf16":
                return t.double()
            inv = codecs.inverse_scale(sc)
            return (t.float() * float(inv)).clamp(-448, 448).to(torch.float8_e4m3fn).double() * float(np.float32(sc))
        K = dec(case.seq_k(s), case.k_scale).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        V = dec(case.seq_v(s), case.v_scale).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q.reshape(1, -1, 1, D), K, V, scale=case.scale)
        assert np.max(np.abs(got[s] - ref[0, :, 0].numpy())) < 1e-11
