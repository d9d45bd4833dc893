"""Pins for the oracle's codecs (CPU only): bf16 and fp8 e4m3fn against torch's casts
and against hand-written codes from the OCP 8-bit float definition."""
import json
import os

import numpy as np
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.json")


def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_bf16_decode_all_codes_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(codecs.bf16_to_f64(bits), ref)


def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(codecs.e4m3fn_to_f64(codes), ref)
    assert codecs.E4M3FN_TABLE[0x7E] == 448.0 and np.isnan(codecs.E4M3FN_TABLE[0x7F])


def test_quantiser_hand_written_codes():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    x = np.array([c[0] for c in cases], dtype=np.float32)
    want = np.array([c[1] for c in cases], dtype=np.uint8)
    got = codecs.quantize_e4m3fn(x, np.float32(1.0))
    bad = [(float(a), int(b), int(c)) for a, b, c in zip(x, got, want) if b != c]
    assert not bad, bad


def test_quantiser_matches_torch_in_range():
    rng = np.random.default_rng(0)
    # Magnitudes across the whole range, including subnormals, plus exact grid midpoints.
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), size=200_000)).astype(np.float32)
    x = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    grid = codecs.E4M3FN_TABLE[:0x7F]
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, grid.astype(np.float32)])
    inv = np.float32(1.0)
    got = codecs.quantize_e4m3fn(x, inv)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_quantiser_scale_is_one_float32_multiply():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50_000).astype(np.float32)
    scale = np.float32(np.max(np.abs(x)) / np.float32(448.0))
    inv = codecs.inverse_scale(scale)
    assert inv == np.float32(np.float32(1.0) / scale)
    got = codecs.quantize_e4m3fn(x, inv)
    ref = torch.from_numpy((x * inv).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert np.array_equal(got, ref.view(torch.uint8).numpy())
    # Dequantised values lie within half an fp8 step of the scaled input.
    deq = codecs.e4m3fn_to_f64(got) * np.float64(scale)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2 ** -4 + scale * 2 ** -10 + 1e-12)


def test_bf16_input_quantiser_goes_through_exact_float32():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10_000).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    f = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    inv = np.float32(37.5)
    assert np.array_equal(codecs.quantize_bf16_to_e4m3fn(bits, inv), codecs.quantize_e4m3fn(f, inv))


def test_quantiser_table_equals_the_per_element_quantiser():
    """The per-code table the oracle looks fp8 codes up in holds exactly what the quantiser
    gives for each bf16 input, at several scales, on random bf16 values including NaN,
    infinities, huge and subnormal ones."""
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=200_000).astype(np.uint16)
    for scale in (1.0, 0.0123, 4.5 / 448, 3.3e-5):
        inv = codecs.inverse_scale(scale)
        table = codecs.bf16_to_e4m3fn_table(inv)
        assert table.dtype == np.uint8 and table.shape == (1 << 16,)
        assert np.array_equal(table[bits], codecs.quantize_bf16_to_e4m3fn(bits, inv))
