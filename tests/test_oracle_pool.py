"""Pins for the oracle's pool model (CPU only): layout structure, write/gather, copy."""
import itertools

import numpy as np
import pytest

from oracle import codecs
from oracle import pool as opool
from synth import bf16_bits_from_f32

COMBOS = [(dt, D, bs) for dt in ("f32", "bf16", "fp8_e4m3fn") for D in (64, 128) for bs in (16, 32)]


@pytest.mark.parametrize("dt,D,bs", COMBOS)
def test_offsets_are_a_permutation_of_each_region(dt, D, bs):
    for offs in (opool.k_offsets(bs, D, dt), opool.v_offsets(bs, D, dt)):
        assert np.array_equal(np.sort(offs.ravel()), np.arange(bs * D))


@pytest.mark.parametrize("dt,D,bs", COMBOS)
def test_k_chunk_is_consecutive_dims_of_one_token(dt, D, bs):
    x = 16 // opool.ELEM_BYTES[dt]
    offs = opool.k_offsets(bs, D, dt)
    where = {int(offs[o, d]): (o, d) for o, d in itertools.product(range(bs), range(D))}
    for c in range(bs * D // x):
        members = [where[c * x + i] for i in range(x)]
        toks = {o for o, _ in members}
        dims = [d for _, d in members]
        assert len(toks) == 1
        assert dims == list(range(dims[0], dims[0] + x)) and dims[0] % x == 0


@pytest.mark.parametrize("dt,D,bs", COMBOS)
def test_v_chunk_is_four_consecutive_tokens_for_dims_sixteen_apart(dt, D, bs):
    x = 16 // opool.ELEM_BYTES[dt]
    x4 = x // 4
    offs = opool.v_offsets(bs, D, dt)
    where = {int(offs[o, d]): (o, d) for o, d in itertools.product(range(bs), range(D))}
    for c in range(bs * D // x):
        members = [where[c * x + i] for i in range(x)]
        for e in range(x4):
            run = members[4 * e:4 * e + 4]
            toks = [o for o, _ in run]
            assert toks == list(range(toks[0], toks[0] + 4)) and toks[0] % 4 == 0
            assert len({d for _, d in run}) == 1
        dims = [members[4 * e][1] for e in range(x4)]
        assert dims == [dims[0] + 16 * e for e in range(x4)]
    # Each 16-token sub-tile occupies its own contiguous 16*D run.
    for o in range(bs):
        assert np.all(offs[o] // (16 * D) == o // 16)


def _values(rng, shape, dt):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if dt == "f32" else bf16_bits_from_f32(x)


@pytest.mark.parametrize("dt,D,bs", COMBOS)
def test_write_then_gather_round_trips(dt, D, bs):
    rng = np.random.default_rng(hash((dt, D, bs)) % 2**32)
    NB, Hkv = 9, 3
    in_dt = "bf16" if dt == "fp8_e4m3fn" else dt
    pk = opool.empty_pool(NB, Hkv, bs, D, dt)
    pv = opool.empty_pool(NB, Hkv, bs, D, dt)
    L = 2 * bs + 5
    table = rng.permutation(NB)[:3]
    slots = table[np.arange(L) // bs] * bs + np.arange(L) % bs
    k = _values(rng, (L, Hkv, D), in_dt)
    v = _values(rng, (L, Hkv, D), in_dt)
    opool.write(pk, pv, k, v, slots, in_dt, dt, bs, 0.01, 0.02)
    gk = opool.gather(pk, table, L, bs, D, dt, "k")
    gv = opool.gather(pv, table, L, bs, D, dt, "v")
    assert np.array_equal(gk, opool.encode_tokens(k, in_dt, dt, 0.01))
    assert np.array_equal(gv, opool.encode_tokens(v, in_dt, dt, 0.02))
    if dt == "fp8_e4m3fn":
        assert np.array_equal(gk, codecs.quantize_bf16_to_e4m3fn(k, codecs.inverse_scale(0.01)))


def test_write_touches_only_its_slots_and_skips_negative_slots():
    rng = np.random.default_rng(3)
    NB, Hkv, bs, D = 6, 2, 16, 64
    pk = opool.empty_pool(NB, Hkv, bs, D, "bf16", fill=0xABCD)
    pv = opool.empty_pool(NB, Hkv, bs, D, "bf16", fill=0x1234)
    k = _values(rng, (3, Hkv, D), "bf16")
    v = _values(rng, (3, Hkv, D), "bf16")
    slots = np.array([5 * bs + 7, -1, 2 * bs + 15])
    opool.write(pk, pv, k, v, slots, "bf16", "bf16", bs)
    changed_k = np.argwhere(pk != 0xABCD)
    assert set(map(int, np.unique(changed_k[:, 0]))) <= {5, 2}
    assert np.count_nonzero(pk != 0xABCD) <= 2 * Hkv * D
    assert np.array_equal(opool.gather(pk, [5], 8, bs, D, "bf16", "k")[7], k[0])
    assert np.array_equal(opool.gather(pv, [0, 0, 2], 48, bs, D, "bf16", "v")[47], v[2])


def test_copy_blocks_copies_whole_blocks_and_leaves_sources():
    rng = np.random.default_rng(4)
    pk = rng.integers(0, 2**16, size=(8, 2, 16 * 64), dtype=np.uint16)
    pv = rng.integers(0, 2**16, size=(8, 2, 16 * 64), dtype=np.uint16)
    k0, v0 = pk.copy(), pv.copy()
    opool.copy_blocks(pk, pv, [(1, 4), (6, 0)])
    assert np.array_equal(pk[4], k0[1]) and np.array_equal(pv[0], v0[6])
    for b in (1, 2, 3, 5, 6, 7):
        assert np.array_equal(pk[b], k0[b]) and np.array_equal(pv[b], v0[b])
