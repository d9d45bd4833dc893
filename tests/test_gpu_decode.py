"""Paged decode attention on the GPU against the fp64 oracle.

Sizes here finish in seconds on the oracle yet span several 16-token sub-tiles, several
blocks and ragged tails, with unused slots and blocks poisoned with NaN.  Tolerances:
fp32 max |d| <= 1e-5; bf16 and fp8 |d| <= 2e-2 + 1e-2 |ref| per element.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from synth import WORKLOADS, Workload, bf16_bits_from_f32, make_decode_case

from gpu_helpers import as_f64, assert_close, decode, log, pack, random_decode_case, raw_bytes, require_gpu, to_dev

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "llama3_8b_bf16": WORKLOADS["llama3_8b_bf16"].scaled(batch=6, length_dist=("uniform", 1, 700)),
    "long_ctx_splitk_bf16": WORKLOADS["long_ctx_splitk_bf16"].scaled(batch=2, length_dist=("uniform", 2000, 5000)),
    "fp8_kv": WORKLOADS["fp8_kv"].scaled(batch=4, length_dist=("uniform", 1, 1500)),
    # Other supported shapes: D 64 / bs 32 / G 2, G 16, f32 with D 128 and bs 32, fp8 with D 64,
    # G 6 and G 3.
    "bf16_d64_bs32_g2": Workload("bf16_d64_bs32_g2", 5, 8, 4, 64, 32, "bf16", "bf16", ("uniform", 1, 300)),
    "bf16_g16": Workload("bf16_g16", 3, 32, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 400)),
    "f32_d128_bs32_g4": Workload("f32_d128_bs32_g4", 3, 16, 4, 128, 32, "f32", "f32", ("uniform", 1, 300)),
    "fp8_d64_bs16_g8": Workload("fp8_d64_bs16_g8", 3, 16, 2, 64, 16, "bf16", "fp8_e4m3fn", ("uniform", 1, 500)),
    # Groups that are not a multiple of the merge's four heads per wave: idle lanes.
    "bf16_g6": Workload("bf16_g6", 4, 12, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 900)),
    "f32_d64_g3": Workload("f32_d64_g3", 3, 9, 3, 64, 16, "f32", "f32", ("uniform", 1, 400)),
    # Kv heads walked in groups: 6 heads go in pairs, 16 heads in four groups of four.
    "bf16_hkv6_g2": Workload("bf16_hkv6_g2", 3, 12, 6, 128, 16, "bf16", "bf16", ("uniform", 1, 500)),
    "f32_d64_hkv16_g1": Workload("f32_d64_hkv16_g1", 2, 16, 16, 64, 16, "f32", "f32", ("uniform", 1, 300)),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_parity_small(name, seed):
    require_gpu()
    wl = SMALL[name]
    case = make_decode_case(wl, seed)
    log(f"parity {name} seed={seed} lengths={case.lengths.tolist()}")
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, name)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes(seed):
    require_gpu()
    case, splits = random_decode_case(seed)
    wl = case.wl
    log(f"random decode {seed}: D={wl.head_dim} bs={wl.block_size} kv={wl.kv_dtype} G={wl.group_size} "
        f"Hkv={wl.num_kv_heads} B={wl.batch} splits={splits} lengths={case.lengths.tolist()}")
    k, v = pack(case)
    got = as_f64(decode(case, k, v, num_splits=splits))
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, f"random decode {seed}")


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "long_ctx_splitk_bf16", "tiny_fp32", "fp8_kv", "bf16_hkv6_g2"])
def test_split_count_does_not_change_the_result(name):
    require_gpu()
    wl = SMALL[name]
    case = make_decode_case(wl, 11)
    k, v = pack(case)
    ref = oatt.decode_case(case)
    outs = []
    for n in (1, 2, 3, 4, 7, 64, 1000, 0):
        log(f"splits {name} num_splits={n}")
        got = as_f64(decode(case, k, v, num_splits=n))
        assert_close(got, ref, wl.kv_dtype, f"{name} splits={n}")
        outs.append(got)
    # One share per wave is exact arithmetic order per split count; different counts only
    # regroup the running softmax, so they agree closely with each other too.
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < (1e-5 if wl.kv_dtype == "f32" else 3e-2)


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "fp8_kv", "tiny_fp32"])
def test_physical_block_permutation_is_bit_identical(name):
    """The same logical K/V under a different physical numbering gives identical bits."""
    require_gpu()
    wl = SMALL[name]
    case = make_decode_case(wl, 3)
    k, v = pack(case)
    base = decode(case, k, v)
    rng = np.random.default_rng(99)
    relabel = rng.permutation(case.num_blocks).astype(np.int32)
    tables2 = np.where(case.block_tables >= 0, relabel[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    k2, v2 = pack(case, tables=tables2)
    other = decode(case, k2, v2, tables=tables2)
    assert raw_bytes(base) == raw_bytes(other)


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "tiny_fp32"])
@pytest.mark.parametrize("num_splits", [0, 3000])
def test_long_and_short_sequences_together(name, num_splits):
    """One long sequence beside short and empty ones: the table is wide enough that the
    merge splits each head's pieces over four waves, while the short sequences' heads have
    fewer pieces than waves (some waves fold nothing)."""
    require_gpu()
    wl = SMALL[name].scaled(batch=5)
    lengths = np.array([1800 if wl.kv_dtype != "f32" else 400, 20, 0, 40, 3], dtype=np.int64)
    case = make_decode_case(wl, 6, lengths=lengths)
    log(f"long and short {name} splits={num_splits} lengths={lengths.tolist()}")
    k, v = pack(case)
    got = as_f64(decode(case, k, v, num_splits=num_splits))
    assert np.all(got[2] == 0)
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, name)


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "tiny_fp32", "fp8_kv"])
def test_empty_and_single_token_sequences(name):
    require_gpu()
    wl = SMALL[name].scaled(batch=6)
    lengths = np.array([0, 1, 17, 0, 33, 1], dtype=np.int64)
    case = make_decode_case(wl, 4, lengths=lengths)
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    ref = oatt.decode_case(case)
    assert np.all(got[0] == 0) and np.all(got[3] == 0)
    assert_close(got, ref, wl.kv_dtype, name)
    if wl.kv_dtype != "fp8_e4m3fn":
        # One token: the output is that token's value exactly (weight 1, sum 1).
        G = wl.group_size
        for s in (1, 5):
            vals = oatt.kv_to_f64(case.seq_v(s), wl.kv_dtype)[0]
            for h in range(wl.num_q_heads):
                assert np.array_equal(got[s, h], vals[h // G])


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "fp8_kv", "tiny_fp32"])
@pytest.mark.parametrize("num_splits", [0, 7, 64])
def test_many_short_sequences(name, num_splits):
    """A batch of 300 short sequences (some empty): the per-sequence work offsets are
    scanned over five 64-sequence chunks, and one share walks many whole units."""
    require_gpu()
    wl = SMALL[name].scaled(batch=300, length_dist=("uniform", 0, 40), pool_blocks=None)
    case = make_decode_case(wl, 12)
    log(f"many short {name} splits={num_splits} sum L={int(case.lengths.sum())}")
    k, v = pack(case)
    got = as_f64(decode(case, k, v, num_splits=num_splits))
    assert np.all(got[case.lengths == 0] == 0)
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, f"{name} splits={num_splits}")


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "tiny_fp32"])
@pytest.mark.parametrize("batch", [512, 520])
def test_batches_around_the_scan_limit(name, batch):
    """The split pass scans batches of up to 512 sequences into LDS in every workgroup and
    walks larger ones wave by wave: a batch at the limit and one past it, short sequences
    with empty ones among them, against the oracle."""
    require_gpu()
    wl = SMALL[name].scaled(batch=batch, length_dist=("uniform", 0, 60), pool_blocks=None)
    case = make_decode_case(wl, 13)
    log(f"batch {batch} {name} sum L={int(case.lengths.sum())}")
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    assert np.all(got[case.lengths == 0] == 0)
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, f"{name} batch {batch}")


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "fp8_kv", "tiny_fp32"])
@pytest.mark.parametrize("num_splits", [0, 5])
def test_context_lengths_outside_the_table_are_clamped(name, num_splits):
    """context_lens past max_blocks_per_seq * bs read the full table row, and a negative
    length reads as an empty sequence (zero output), as the boundary states."""
    require_gpu()
    wl = SMALL[name].scaled(batch=4)
    bs = wl.block_size
    lengths = np.array([20 * bs, 50, 3 * bs + 7, 9], dtype=np.int64)   # row 0 fills the table
    case = make_decode_case(wl, 8, lengths=lengths)
    assert case.block_tables.shape[1] * bs == lengths[0]
    k, v = pack(case)
    passed = lengths.copy()
    passed[0] = lengths[0] + 37       # past the table row: clamped to its 20 blocks
    passed[3] = -5                    # negative: no tokens
    got = as_f64(decode(case, k, v, num_splits=num_splits, lengths=passed))
    ref = oatt.decode_case(case)
    assert np.all(got[3] == 0)
    assert_close(got[:3], ref[:3], wl.kv_dtype, f"{name} splits={num_splits}")


def test_all_sequences_empty():
    require_gpu()
    wl = SMALL["llama3_8b_bf16"].scaled(batch=3)
    case = make_decode_case(wl, 5, lengths=np.zeros(3, dtype=np.int64))
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    assert np.all(got == 0)


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "long_ctx_splitk_bf16"])
def test_large_logits(name):
    """q scaled by 30: nearly one-hot softmax, no overflow, parity holds."""
    require_gpu()
    wl = SMALL[name]
    case = make_decode_case(wl, 6)
    qf = (case.q.astype(np.uint32) << 16).view(np.float32) * np.float32(30.0)
    case.q = bf16_bits_from_f32(qf)
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    assert_close(got, oatt.decode_case(case), wl.kv_dtype, name)


def test_unpoisoned_pool_gives_the_same_bits():
    require_gpu()
    wl = SMALL["llama3_8b_bf16"]
    case = make_decode_case(wl, 7)
    k, v = pack(case, poison=True)
    k0, v0 = pack(case, poison=False)
    a = raw_bytes(decode(case, k, v))
    b = raw_bytes(decode(case, k0, v0))
    assert a == b


def test_default_split_count_does_not_depend_on_the_hint():
    """num_splits = 0 picks the same split count with or without shared-prefix counts: the
    default workspace is that of the default count, and a hinted call at the default gives
    the same output bits as a plain one."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    for kd, bs in ((pkv.BF16, 16), (pkv.FP8_E4M3FN, 32)):
        d = pkv.paged_attention_default_splits(128, bs, pkv.BF16, kd)
        ws0 = pkv.paged_attention_workspace_size(64, 32, 8, 128, bs, pkv.BF16, kd, 0)
        assert ws0 == pkv.paged_attention_workspace_size(64, 32, 8, 128, bs, pkv.BF16, kd, d)
    case = make_decode_case(SMALL["llama3_8b_bf16"], 4)
    k, v = pack(case)
    counts = np.random.default_rng(4).integers(-1, case.block_tables.shape[1] + 2, size=case.wl.batch)
    assert raw_bytes(decode(case, k, v)) == raw_bytes(decode(case, k, v, shared_prefix_blocks=counts))


def _split_then_reduce(case, k, v, split_kw, reduce_kw, ws):
    import paged_kv_cache_329_amd as pkv
    wl = case.wl
    q = to_dev(case.q, wl.q_dtype)
    out = torch.full_like(q, 7.0)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).cuda()
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    pkv.paged_attention_split(out, q, k, v, tables, lens, case.scale, workspace=ws, **split_kw)
    pkv.paged_attention_reduce(out, q, k, v, tables, lens, case.scale, workspace=ws, **reduce_kw)
    torch.cuda.synchronize()
    return out


def test_reduce_follows_the_split_pass_record():
    """The reduce pass takes the split count and head grouping from the header the split
    pass wrote at the start of the workspace: a reduce given another num_splits or other
    shared-prefix counts still merges what the split pass left (the oracle's result), and
    with the split pass's num_splits gives the one-call decode's bits."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    case = make_decode_case(SMALL["llama3_8b_bf16"], 5)
    k, v = pack(case)
    wl = case.wl
    ws = torch.zeros(pkv.paged_attention_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                        wl.block_size, pkv.BF16, pkv.BF16, 640),
                     dtype=torch.uint8, device="cuda")
    counts = torch.from_numpy(np.full(wl.batch, 2, np.int32)).cuda()
    want = decode(case, k, v, num_splits=640)
    ref = oatt.decode_case(case)
    for split_kw, reduce_kw in (({"num_splits": 640}, {"num_splits": 640}),
                                ({"num_splits": 640, "shared_prefix_blocks": counts}, {"num_splits": 640}),
                                ({"num_splits": 640, "shared_prefix_blocks": counts}, {"num_splits": 0}),
                                ({"num_splits": 640}, {"num_splits": 3, "shared_prefix_blocks": counts})):
        got = _split_then_reduce(case, k, v, split_kw, reduce_kw, ws)
        assert_close(as_f64(got), ref, wl.kv_dtype, f"split {split_kw} then reduce {reduce_kw}")
        if reduce_kw["num_splits"] == 640:
            # Same merge kernel as the one-call decode: the same bits.
            assert raw_bytes(got) == raw_bytes(want), (split_kw, reduce_kw)
        else:
            # Another split count may pick the other merge variant (a different fold order):
            # the same partials, merged within a bf16 rounding of the one-call result.
            d = np.abs(as_f64(got) - as_f64(want))
            assert np.all(d <= 2.0 ** -7 * np.abs(as_f64(want)) + 1e-6), (split_kw, reduce_kw, d.max())


def test_reduce_without_a_split_pass_writes_nan():
    """A reduce pass over a workspace that no split pass over these sequences wrote (here
    zeroed) follows nothing in it and writes NaN into the heads it merges, so the mistake
    shows; the sequences' other heads are untouched."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    case = make_decode_case(SMALL["llama3_8b_bf16"], 5)
    k, v = pack(case)
    wl = case.wl
    q = to_dev(case.q, wl.q_dtype)
    out = torch.zeros_like(q)
    ws = torch.zeros(pkv.paged_attention_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                        wl.block_size, pkv.BF16, pkv.BF16, 640),
                     dtype=torch.uint8, device="cuda")
    pkv.paged_attention_reduce(out, q, k, v, torch.from_numpy(np.ascontiguousarray(case.block_tables)).cuda(),
                               torch.from_numpy(case.lengths.astype(np.int32)).cuda(), case.scale,
                               num_splits=640, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
