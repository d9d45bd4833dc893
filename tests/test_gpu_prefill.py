"""Causal multi-query paged attention (prefill, prefill chunks, drafted-token checks) on the
GPU against the fp64 oracle.

Small cases finish in seconds on the oracle yet span several 16-token sub-tiles, several
staging steps and query tiles, ragged tails and partial column tiles, with unused slots and
blocks poisoned with NaN.  Tolerances as for decode: fp32 max |d| <= 1e-5; bf16 and fp8
|d| <= 2e-2 + 1e-2 |ref| per element.
"""
import numpy as np
import pytest

from oracle import attention as oatt
from synth import WORKLOADS, Workload, make_prefill_case

from gpu_helpers import (as_f64, assert_close, decode, log, pack, prefill, prefill_default_order, raw_bytes,
                         require_gpu, to_dev)

pytestmark = pytest.mark.gpu

SMALL = {
    "prefill_tiny_fp32": WORKLOADS["prefill_tiny_fp32"],
    "prefill_bf16": WORKLOADS["prefill_llama3_8b_bf16"].scaled(batch=3, length_dist=("uniform", 1, 300)),
    "chunk_bf16": WORKLOADS["chunked_prefill_llama3_8b_bf16"].scaled(
        batch=4, length_dist=("uniform", 1, 400), query_dist=("fixed", 70)),
    "verify_bf16": WORKLOADS["spec_verify_llama3_8b_bf16"].scaled(batch=6, length_dist=("uniform", 1, 500)),
    "prefill_fp8": WORKLOADS["prefill_fp8_kv"].scaled(batch=3, length_dist=("uniform", 1, 300)),
    # Other shapes: D 64 / bs 32 / G 2, G 16, G 1, G 3 (column tiles cross query tokens),
    # f32 with D 128 and bs 32, fp8 with D 64 and with D 128 / bs 16.
    "bf16_d64_bs32_g2": Workload("bf16_d64_bs32_g2", 3, 8, 4, 64, 32, "bf16", "bf16", ("uniform", 1, 200),
                                 query_dist=("fixed", 50)),
    "bf16_g16": Workload("bf16_g16", 2, 32, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 150),
                         query_dist=("all",)),
    "bf16_g1": Workload("bf16_g1", 2, 4, 4, 128, 16, "bf16", "bf16", ("uniform", 60, 260),
                        query_dist=("all",)),
    "bf16_g3": Workload("bf16_g3", 3, 6, 2, 64, 16, "bf16", "bf16", ("uniform", 1, 120),
                        query_dist=("fixed", 33)),
    "f32_d128_bs32_g4": Workload("f32_d128_bs32_g4", 2, 16, 4, 128, 32, "f32", "f32", ("uniform", 1, 150),
                                 query_dist=("all",)),
    "fp8_d64_bs16_g8": Workload("fp8_d64_bs16_g8", 3, 16, 2, 64, 16, "bf16", "fp8_e4m3fn", ("uniform", 1, 200),
                                query_dist=("fixed", 40)),
    # fp8 widened to bf16 at staging: D 128 with 16-token blocks as well.
    "fp8_d128_bs16_g2": Workload("fp8_d128_bs16_g2", 3, 8, 4, 128, 16, "bf16", "fp8_e4m3fn", ("uniform", 1, 250),
                                 query_dist=("fixed", 40)),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("seed", [0, 1])
def test_parity_small(name, seed):
    require_gpu()
    wl = SMALL[name]
    case = make_prefill_case(wl, seed)
    log(f"prefill parity {name} seed={seed} lengths={case.lengths.tolist()} q_lens={case.q_lens.tolist()}")
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    assert_close(got, oatt.prefill_case(case), wl.kv_dtype, name)


def test_edge_query_counts():
    """n_s = 0, n_s = L_s, n_s > L_s (the first queries sit before position 0: zeros),
    L_s = 0, a single token, and lengths on sub-tile and step boundaries."""
    require_gpu()
    wl = SMALL["prefill_bf16"].scaled(batch=9)
    lengths = np.array([5, 16, 64, 65, 1, 0, 31, 128, 3])
    q_lens = np.array([0, 16, 10, 65, 1, 2, 40, 1, 7])
    case = make_prefill_case(wl, 3, lengths=lengths, q_lens=q_lens)
    log(f"prefill edges lengths={lengths.tolist()} q_lens={q_lens.tolist()}")
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    ref = oatt.prefill_case(case)
    assert_close(got, ref, wl.kv_dtype, "edges")
    qs = case.query_start
    assert np.all(got[qs[5]:qs[6]] == 0)            # L = 0: no keys at all
    assert np.all(got[qs[6]:qs[6] + 9] == 0)        # n = 40 > L = 31: first 9 queries see nothing


def test_max_query_len_bounds_the_rows_written():
    require_gpu()
    wl = SMALL["chunk_bf16"]
    case = make_prefill_case(wl, 4)
    k, v = pack(case)
    cap = 20
    got = prefill(case, k, v, max_query_len=cap)
    full = prefill(case, k, v)
    qs = case.query_start
    for s in range(wl.batch):
        a, b = int(qs[s]), int(qs[s + 1])
        m = min(b - a, cap)
        assert raw_bytes(got[a:a + m]) == raw_bytes(full[a:a + m])


def test_one_query_per_sequence_matches_decode():
    require_gpu()
    wl = SMALL["verify_bf16"].scaled(query_dist=("one",), length_dist=("uniform", 1, 900))
    case = make_prefill_case(wl, 5)
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    dec = as_f64(decode(case, k, v, q=case.q))
    assert_close(got, oatt.prefill_case(case), wl.kv_dtype, "prefill n=1")
    assert np.max(np.abs(got - dec)) <= 2e-2


def test_chunks_and_block_placement_do_not_change_bits():
    """Each output column runs the same arithmetic whatever the other queries of its tile
    and wherever the blocks sit: the queries computed in two chunks (the first over the
    tokens that exist when it runs) and over a permuted pool give the same bytes."""
    require_gpu()
    wl = SMALL["prefill_bf16"].scaled(batch=2, length_dist=("uniform", 150, 300))
    case = make_prefill_case(wl, 6)
    k, v = pack(case)
    whole = prefill(case, k, v)
    qs = case.query_start
    for s in range(wl.batch):
        L = int(case.lengths[s])
        a = int(qs[s])
        split = 37 + 20 * s
        one = make_prefill_case(wl.scaled(batch=1), 6, lengths=[L], q_lens=[L])
        one.q = case.q[a:a + L]
        one.k, one.v = case.seq_k(s), case.seq_v(s)
        one.offsets = np.array([0, L])
        ko, vo = pack(one)
        first = prefill(one, ko, vo, lengths=[split], query_start=[0, split], q=one.q[:split])
        second = prefill(one, ko, vo, query_start=[0, L - split], q=one.q[split:])
        assert raw_bytes(first) == raw_bytes(whole[a:a + split])
        assert raw_bytes(second) == raw_bytes(whole[a + split:a + L])
    # A different physical placement of the same logical blocks.
    rng = np.random.default_rng(0)
    perm = rng.permutation(case.num_blocks)
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    k2, v2 = pack(case, tables=tables)
    assert raw_bytes(prefill(case, k2, v2, tables=tables)) == raw_bytes(whole)


def test_large_logits_stay_finite():
    require_gpu()
    wl = SMALL["prefill_bf16"]
    case = make_prefill_case(wl, 7)
    q32 = case.q.view(np.uint16).astype(np.uint32) << 16
    big = (q32.view(np.float32) * 30.0).astype(np.float32)
    import torch
    case.q = torch.from_numpy(big).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    assert_close(got, oatt.prefill_case(case), wl.kv_dtype, "large logits")


# ---- the few-query path (max_query_len * G <= 32): shares over the keys, then a merge ----

FEW = {
    "f32_d64_g2_n16": Workload("f32_d64_g2_n16", 4, 8, 4, 64, 16, "f32", "f32", ("uniform", 1, 300),
                               query_dist=("fixed", 16)),
    "bf16_g4_n8": Workload("bf16_g4_n8", 6, 32, 8, 128, 16, "bf16", "bf16", ("uniform", 1, 700),
                           query_dist=("fixed", 8)),
    "fp8_g4_n8": Workload("fp8_g4_n8", 4, 32, 8, 128, 32, "bf16", "fp8_e4m3fn", ("uniform", 1, 900),
                          query_dist=("fixed", 8)),
    "bf16_d64_bs32_g8_n4": Workload("bf16_d64_bs32_g8_n4", 5, 16, 2, 64, 32, "bf16", "bf16",
                                    ("uniform", 1, 500), query_dist=("fixed", 4)),
    "bf16_g16_n2": Workload("bf16_g16_n2", 3, 32, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 400),
                            query_dist=("fixed", 2)),
    "bf16_g1_n32": Workload("bf16_g1_n32", 3, 4, 4, 128, 16, "bf16", "bf16", ("uniform", 1, 400),
                            query_dist=("fixed", 32)),
    # 15 columns: the merge wave of columns 12..15 has one idle column of lanes.
    "bf16_g3_n5": Workload("bf16_g3_n5", 4, 6, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 600),
                           query_dist=("fixed", 5)),
}


@pytest.mark.parametrize("name", list(FEW))
@pytest.mark.parametrize("splits", [0, 3, 5, 997])
def test_few_query_path_parity(name, splits):
    require_gpu()
    import torch
    import paged_kv_cache_329_amd as pkv
    wl = FEW[name]
    case = make_prefill_case(wl, 2)
    log(f"few-query {name} splits={splits} lengths={case.lengths.tolist()} q_lens={case.q_lens.tolist()}")
    k, v = pack(case)
    q = to_dev(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, k, v, torch.from_numpy(case.block_tables).cuda(),
                                torch.from_numpy(case.lengths.astype(np.int32)).cuda(),
                                torch.from_numpy(case.query_start).cuda(), int(case.q_lens.max()), case.scale,
                                float(case.k_scale), float(case.v_scale), num_splits=splits)
    torch.cuda.synchronize()
    assert_close(as_f64(out), oatt.prefill_case(case), wl.kv_dtype, name)


@pytest.mark.parametrize("splits", [0, 7])
def test_few_query_path_many_short_sequences(splits):
    """200 short sequences with 0..5 queries each (lengths 0..60, so some queries sit before
    position 0): many units per share, and sequence offsets over several 64-entry chunks."""
    require_gpu()
    wl = FEW["bf16_g4_n8"].scaled(batch=200, length_dist=("uniform", 0, 60))
    rng = np.random.default_rng(31)
    lengths = rng.integers(0, 61, size=200)
    q_lens = rng.integers(0, 6, size=200)
    case = make_prefill_case(wl, 9, lengths=lengths, q_lens=q_lens)
    log(f"few-query many short splits={splits} queries={int(q_lens.sum())}")
    k, v = pack(case)
    assert int(case.q_lens.max()) * wl.group_size <= 32
    got = as_f64(prefill(case, k, v) if splits == 0 else _prefill_splits(case, k, v, splits))
    assert_close(got, oatt.prefill_case(case), wl.kv_dtype, f"few-query many short splits={splits}")


ORDER_CASES = {
    # Many (sequence, kv head) units per XCD with unequal lengths, several tiles each.
    "prefill_bf16": WORKLOADS["prefill_llama3_8b_bf16"].scaled(batch=14, length_dist=("uniform", 1, 700)),
    "chunk_bf16": WORKLOADS["chunked_prefill_llama3_8b_bf16"].scaled(
        batch=12, length_dist=("uniform", 1, 900), query_dist=("fixed", 150)),
    "prefill_fp8": WORKLOADS["prefill_fp8_kv"].scaled(batch=10, length_dist=("uniform", 1, 600)),
    "f32_d128_bs32_g4": SMALL["f32_d128_bs32_g4"].scaled(batch=9, length_dist=("uniform", 1, 400)),
}


@pytest.mark.parametrize("name", list(ORDER_CASES))
def test_tile_path_launch_order_leaves_the_bits(name):
    """The tile path with a workspace first runs a plan pass that launches the query tiles
    longest first; without one (NULL) they run in the default order.  Both give the oracle's
    result and the same bytes, and the plan needs no initial workspace contents (it is
    poisoned with 0xFF bytes first)."""
    require_gpu()
    import torch
    import paged_kv_cache_329_amd as pkv
    wl = ORDER_CASES[name]
    case = make_prefill_case(wl, 6)
    log(f"launch order {name} lengths={case.lengths.tolist()} q_lens={case.q_lens.tolist()}")
    k, v = pack(case)
    q = to_dev(case.q, wl.q_dtype)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).cuda()
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    qs = torch.from_numpy(case.query_start.astype(np.int32)).cuda()
    max_q = int(case.q_lens.max())
    G = wl.num_q_heads // wl.num_kv_heads
    assert max_q * G > pkv.FEW_QUERY_COLUMNS                 # the tile path
    qd = pkv.F32 if wl.q_dtype == "f32" else pkv.BF16
    kd = {"f32": pkv.F32, "bf16": pkv.BF16, "fp8_e4m3fn": pkv.FP8_E4M3FN}[wl.kv_dtype]
    nbytes = pkv.paged_attention_prefill_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                         wl.block_size, qd, kd, max_q, 0)
    assert nbytes > 0
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    planned = torch.empty_like(q)
    pkv.paged_attention_prefill(planned, q, k, v, tables, lens, qs, max_q, case.scale, float(case.k_scale),
                                float(case.v_scale), workspace=ws)
    torch.cuda.synchronize()
    assert_close(as_f64(planned), oatt.prefill_case(case), wl.kv_dtype, f"launch order {name}")
    assert raw_bytes(prefill_default_order(case, k, v)) == raw_bytes(planned)


def _random_tile_case(seed):
    """A seeded random tile-path batch: head size, block size, cache type, group size, kv
    heads, batch and lengths, with query counts from a single token up to the whole context."""
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    kv = str(rng.choice(["f32", "bf16", "fp8_e4m3fn"]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 5, 8]))
    B = int(rng.integers(1, 24))
    lengths = rng.integers(0, 500, size=B)
    q_lens = np.minimum(lengths, rng.integers(0, 200, size=B))
    q_lens[rng.integers(0, B)] = max(int(q_lens.max()), 40)            # the tile path
    q_dtype = "f32" if kv == "f32" else "bf16"
    wl = Workload(f"rand{seed}", B, Hkv * G, Hkv, D, bs, q_dtype, kv, ("uniform", 1, 500), query_dist=("all",))
    return make_prefill_case(wl, seed, lengths=np.maximum(lengths, q_lens), q_lens=q_lens)


@pytest.mark.parametrize("seed", range(6))
def test_tile_path_launch_plan_random_shapes(seed):
    """Random shapes through the tile path: the planned launch (the binding's default) gives
    the oracle's result on every row, and the same bytes as the default order (NULL
    workspace)."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    case = _random_tile_case(seed)
    wl = case.wl
    max_q = int(case.q_lens.max())
    assert max_q * wl.group_size > pkv.FEW_QUERY_COLUMNS
    log(f"random tile case {seed}: D={wl.head_dim} bs={wl.block_size} kv={wl.kv_dtype} G={wl.group_size} "
        f"Hkv={wl.num_kv_heads} B={wl.batch} q_lens={case.q_lens.tolist()}")
    k, v = pack(case)
    planned = prefill(case, k, v)
    assert_close(as_f64(planned), oatt.prefill_case(case), wl.kv_dtype, f"random tile case {seed}")
    assert raw_bytes(prefill_default_order(case, k, v)) == raw_bytes(planned)


@pytest.mark.parametrize("name", ["prefill_bf16", "chunk_bf16", "f32_d128_bs32_g4"])
def test_launch_plan_records(name):
    """The plan the tile path leaves in its workspace: one 32-byte record (unit, tile, q0, n,
    L, steps, 0, 0) per workgroup slot, [8 XCDs][units per XCD x tiles].  On each XCD the
    live slots hold exactly the live tiles of the units dealt to it (unit % 8), each unit's
    tiles in one run, last tile first; the runs come in non-increasing order of their first
    (longest) tile's steps; the remaining slots are empty (unit -1); and every record holds
    its sequence's query range and length and its tile's step count."""
    require_gpu()
    import torch
    import paged_kv_cache_329_amd as pkv
    wl = ORDER_CASES[name]
    case = make_prefill_case(wl, 8)
    k, v = pack(case)
    max_q = int(case.q_lens.max())
    qd = pkv.F32 if wl.q_dtype == "f32" else pkv.BF16
    kd = {"f32": pkv.F32, "bf16": pkv.BF16, "fp8_e4m3fn": pkv.FP8_E4M3FN}[wl.kv_dtype]
    nbytes = pkv.paged_attention_prefill_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                         wl.block_size, qd, kd, max_q)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(to_dev(case.q, wl.q_dtype))
    pkv.paged_attention_prefill(out, to_dev(case.q, wl.q_dtype), k, v,
                                torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).cuda(),
                                torch.from_numpy(case.lengths.astype(np.int32)).cuda(),
                                torch.from_numpy(case.query_start.astype(np.int32)).cuda(), max_q, case.scale,
                                float(case.k_scale), float(case.v_scale), workspace=ws)
    torch.cuda.synchronize()
    # Expected geometry, from the documented tiling: 256 (query, head) columns per tile (128
    # for f32), 16 * sub-tiles-per-step keys per step (16 KiB of K per step, at most 8 sub-tiles).
    G, Hkv, B = wl.group_size, wl.num_kv_heads, wl.batch
    cols = 128 if wl.kv_dtype == "f32" else 256
    eb = 4 if wl.kv_dtype == "f32" else 2
    step_tok = 16 * min(8, 16384 // (16 * wl.head_dim * eb))
    tiles = -(-max_q * G // cols)
    per_xcd = -(-B * Hkv // 8) * tiles
    rec = ws[:8 * per_xcd * 32].cpu().numpy().view(np.int32).reshape(8, per_xcd, 8)
    qs = case.query_start.astype(np.int64)
    for x in range(8):
        live = []
        for u in range(x, B * Hkv, 8):
            s_ = u // Hkv
            n, L = int(qs[s_ + 1] - qs[s_]), int(case.lengths[s_])
            for t in range(min(-(-n * G // cols), tiles)):
                last_q = min(n - 1, (t * cols + cols - 1) // G)
                live.append((u, t, int(qs[s_]), n, L, -(-max(L - n + last_q + 1, 0) // step_tok)))
        got = [tuple(int(c) for c in r[:6]) for r in rec[x] if r[0] >= 0]
        assert sorted(got) == sorted(live), f"XCD {x}: the live slots are not the live tiles"
        assert np.all(rec[x][len(got):, 0] == -1) and np.all(rec[x][:len(got), 0] >= 0)
        runs = []
        for r in got:
            if not runs or runs[-1][0][0] != r[0]:
                runs.append([r])
            else:
                runs[-1].append(r)
        assert len({r[0][0] for r in runs}) == len(runs), f"XCD {x}: a unit's tiles are split"
        for run in runs:
            assert [r[1] for r in run] == sorted((r[1] for r in run), reverse=True)
        firsts = [run[0][5] for run in runs]
        assert firsts == sorted(firsts, reverse=True), f"XCD {x}: units not longest first"


def test_tile_path_plan_with_tables_at_the_width_limit():
    """Tables padded to 16,376 entries (the tile path's limit) make the longest possible tile
    4,094 steps, so the plan counts steps in coarser buckets (shifted right by one).  The
    planned and the unplanned launch agree with the oracle and with each other bit for bit."""
    require_gpu()
    wl = ORDER_CASES["prefill_bf16"]
    case = make_prefill_case(wl, 7)
    width = 16376
    tables_np = np.full((wl.batch, width), -1, np.int32)
    tables_np[:, :case.block_tables.shape[1]] = case.block_tables
    k, v = pack(case)
    planned = prefill(case, k, v, tables=tables_np)
    assert_close(as_f64(planned), oatt.prefill_case(case), wl.kv_dtype, "plan at the table width limit")
    assert raw_bytes(prefill_default_order(case, k, v, tables=tables_np)) == raw_bytes(planned)


def test_tile_path_without_a_plan_beyond_its_unit_limit():
    """2,100 short prompts x 8 kv heads is 16,800 (sequence, kv head) units, past the 16,384
    the launch plan orders: the workspace size is 0 and the tiles run in the default order.
    Sampled query rows are checked against the oracle, and every row is finite."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    wl = WORKLOADS["prefill_llama3_8b_bf16"].scaled(batch=2100, length_dist=("uniform", 9, 16))
    case = make_prefill_case(wl, 12)
    max_q = int(case.q_lens.max())
    assert max_q * wl.group_size > pkv.FEW_QUERY_COLUMNS
    assert pkv.paged_attention_prefill_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                      wl.block_size, pkv.BF16, pkv.BF16, max_q) == 0
    log(f"no-plan prefill: {wl.batch} sequences, {case.num_q_tokens} query rows")
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    assert np.all(np.isfinite(got))
    rows = np.sort(np.random.default_rng(3).choice(case.num_q_tokens, size=400, replace=False))
    assert_close(got[rows], oatt.prefill_case(case, rows), wl.kv_dtype, "no-plan prefill")


def _random_few_case(seed):
    """A seeded random few-query batch: at most 32 (query, head) columns per (sequence, kv
    head), over random head and block sizes, cache types, group and batch sizes."""
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    kv = str(rng.choice(["f32", "bf16", "fp8_e4m3fn"]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 40))
    lengths = rng.integers(0, 900, size=B)
    q_lens = np.minimum(rng.integers(0, 32 // G + 1, size=B), np.maximum(lengths, 1))
    q_dtype = "f32" if kv == "f32" else "bf16"
    wl = Workload(f"few{seed}", B, Hkv * G, Hkv, D, bs, q_dtype, kv, ("uniform", 0, 900), query_dist=("all",))
    splits = int(rng.choice([0, 1, 3, 50, 600]))
    return make_prefill_case(wl, seed, lengths=np.maximum(lengths, q_lens), q_lens=q_lens), splits


@pytest.mark.parametrize("seed", range(6))
def test_few_query_path_random_shapes(seed):
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    case, splits = _random_few_case(seed)
    wl = case.wl
    assert int(case.q_lens.max()) * wl.group_size <= pkv.FEW_QUERY_COLUMNS
    log(f"random few-query {seed}: D={wl.head_dim} bs={wl.block_size} kv={wl.kv_dtype} G={wl.group_size} "
        f"Hkv={wl.num_kv_heads} B={wl.batch} splits={splits} q_lens={case.q_lens.tolist()}")
    k, v = pack(case)
    got = as_f64(prefill(case, k, v) if splits == 0 else _prefill_splits(case, k, v, splits))
    assert_close(got, oatt.prefill_case(case), wl.kv_dtype, f"random few-query {seed}")


@pytest.mark.parametrize("B", [512, 520])
def test_few_query_path_batch_sizes_around_the_scan_limit(B):
    """The few-query split pass scans batches of up to 512 sequences into LDS in every
    workgroup and walks larger ones wave by wave: a batch at the limit and one past it, with
    empty sequences and sequences without queries among them, against the oracle."""
    require_gpu()
    import paged_kv_cache_329_amd as pkv
    rng = np.random.default_rng(3100 + B)
    lengths = rng.integers(0, 120, size=B)
    q_lens = np.minimum(rng.integers(0, 9, size=B), lengths)
    wl = Workload(f"few_b{B}", B, 32, 8, 128, 16, "bf16", "bf16", ("uniform", 0, 120), query_dist=("all",))
    case = make_prefill_case(wl, 7, lengths=lengths, q_lens=q_lens)
    assert int(case.q_lens.max()) * wl.group_size <= pkv.FEW_QUERY_COLUMNS
    k, v = pack(case)
    assert_close(as_f64(prefill(case, k, v)), oatt.prefill_case(case), "bf16", f"few-query batch {B}")


def _prefill_splits(case, k, v, splits):
    import torch
    import paged_kv_cache_329_amd as pkv
    wl = case.wl
    q = to_dev(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, k, v, torch.from_numpy(case.block_tables).cuda(),
                                torch.from_numpy(case.lengths.astype(np.int32)).cuda(),
                                torch.from_numpy(case.query_start).cuda(), int(case.q_lens.max()), case.scale,
                                float(case.k_scale), float(case.v_scale), num_splits=splits)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["bf16_g4_n8", "fp8_g4_n8", "f32_d64_g2_n16"])
def test_few_query_path_shared_block_loads_give_the_same_bits(name):
    require_gpu()
    wl = FEW[name]
    case = make_prefill_case(wl, 4)
    k, v = pack(case)
    a = prefill(case, k, v)
    counts = np.random.default_rng(5).integers(-1, case.block_tables.shape[1] + 2, size=wl.batch)
    b = prefill(case, k, v, shared_prefix_blocks=counts)
    assert raw_bytes(a) == raw_bytes(b)


def test_few_query_path_edges_and_placement():
    """n > L (the first queries see nothing), L = 0, n = 0, single tokens; and the same
    bytes when the blocks sit elsewhere in the pool."""
    require_gpu()
    wl = FEW["bf16_g4_n8"].scaled(batch=7)
    lengths = np.array([0, 1, 5, 16, 17, 300, 40])
    q_lens = np.array([1, 3, 5, 2, 8, 8, 0])
    case = make_prefill_case(wl, 8, lengths=lengths, q_lens=q_lens)
    k, v = pack(case)
    got = prefill(case, k, v)
    ref = oatt.prefill_case(case)
    assert_close(as_f64(got), ref, wl.kv_dtype, "few-query edges")
    qs = case.query_start
    assert np.all(as_f64(got)[qs[0]:qs[0] + 1] == 0)          # L = 0
    assert np.all(as_f64(got)[qs[1]:qs[1] + 2] == 0)          # n = 3 > L = 1: positions -2, -1
    rng = np.random.default_rng(1)
    perm = rng.permutation(case.num_blocks)
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    k2, v2 = pack(case, tables=tables)
    assert raw_bytes(prefill(case, k2, v2, tables=tables)) == raw_bytes(got)
