"""Decode attention over contiguous per-sequence placement (pkv_contiguous_attention_decode)
against the fp64 oracle.

Each sequence's blocks are consecutive blocks of an ordinary pool, starting at a first
block of its own with gaps between sequences (poisoned with NaN, as are the unused slots of
each last block).  The kernel computes block addresses from the first block alone
("What is PagedAttention?", glossary, "Common Use Cases": contiguous placement as the
alternative to paging), so the result must be the oracle's, and the same bytes as the paged
kernel reading the same blocks through a table that counts up from the first block.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_329_amd as pkv
from oracle import attention as oatt
from synth import WORKLOADS, Workload, make_decode_case

from gpu_helpers import as_f64, assert_close, decode, pack, raw_bytes, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "llama3_8b_bf16": WORKLOADS["llama3_8b_bf16"].scaled(batch=6, length_dist=("uniform", 0, 900)),
    "fp8_kv": WORKLOADS["fp8_kv"].scaled(batch=4, length_dist=("uniform", 1, 1500)),
    "bf16_g16": Workload("bf16_g16", 3, 32, 2, 128, 16, "bf16", "bf16", ("uniform", 1, 400)),
    "bf16_d64_bs32_g2": Workload("bf16_d64_bs32_g2", 5, 8, 4, 64, 32, "bf16", "bf16", ("uniform", 1, 300)),
}


def _contiguous_tables(case, gap=3):
    """First blocks with `gap` unused blocks before each sequence; tables counting up."""
    bs = case.wl.block_size
    nbs = (case.lengths.astype(np.int64) + bs - 1) // bs
    cap = int(max(1, nbs.max()))
    first = np.zeros(case.wl.batch, dtype=np.int32)
    nxt = gap
    for s in range(case.wl.batch):
        first[s] = nxt
        nxt += int(nbs[s]) + gap
    tables = np.full((case.wl.batch, cap), -1, dtype=np.int32)
    for s in range(case.wl.batch):
        tables[s, :nbs[s]] = first[s] + np.arange(nbs[s])
    return first, tables, nxt


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("num_splits", [0, 37])
def test_contiguous_decode_matches_the_oracle(name, num_splits):
    require_gpu()
    case = make_decode_case(CASES[name], 2)
    first, tables, nb_total = _contiguous_tables(case)
    case.num_blocks = max(case.num_blocks, nb_total)
    k, v = pack(case, tables=tables)
    wl = case.wl
    q = to_dev(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    pkv.contiguous_attention_decode(out, q, k, v, torch.from_numpy(first).cuda(),
                                    torch.from_numpy(case.lengths.astype(np.int32)).cuda(), tables.shape[1],
                                    case.scale, float(case.k_scale), float(case.v_scale), num_splits=num_splits)
    torch.cuda.synchronize()
    assert_close(as_f64(out), oatt.decode_case(case), wl.kv_dtype, f"{name} contiguous")
    assert raw_bytes(out) == raw_bytes(decode(case, k, v, tables=tables, num_splits=num_splits))


def test_contiguous_decode_reads_blocks_outside_the_pool_as_zeros():
    """A first block past the pool: its blocks read as zeros (keys and values), never out of
    bounds, so that sequence's output is zero-key attention over zero values."""
    require_gpu()
    case = make_decode_case(CASES["llama3_8b_bf16"], 3)
    first, tables, nb_total = _contiguous_tables(case)
    case.num_blocks = max(case.num_blocks, nb_total)
    k, v = pack(case, tables=tables)
    wl = case.wl
    bad = first.copy()
    bad[1] = case.num_blocks + 5
    q = to_dev(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    pkv.contiguous_attention_decode(out, q, k, v, torch.from_numpy(bad).cuda(),
                                    torch.from_numpy(case.lengths.astype(np.int32)).cuda(), tables.shape[1],
                                    case.scale)
    torch.cuda.synchronize()
    got = as_f64(out)
    keep = [s for s in range(wl.batch) if s != 1]
    assert_close(got[keep], oatt.decode_case(case, keep), wl.kv_dtype, "other sequences")
    assert np.all(got[1] == 0.0)


def test_contiguous_decode_rejects_bad_arguments():
    require_gpu()
    case = make_decode_case(CASES["llama3_8b_bf16"], 3)
    wl = case.wl
    k, v = pack(case)
    q = to_dev(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    with pytest.raises(ValueError):
        pkv.contiguous_attention_decode(out, q, k, v, torch.zeros(wl.batch + 1, dtype=torch.int32, device="cuda"),
                                        lens, 10, case.scale)
    st = pkv.lib().pkv_contiguous_attention_decode(out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), None,
                                                   lens.data_ptr(), wl.batch, wl.num_q_heads, wl.num_kv_heads,
                                                   wl.head_dim, wl.block_size, k.shape[0], 10, case.scale, 1.0, 1.0,
                                                   pkv.BF16, pkv.BF16, 0, None, 0, None)
    assert st == 1 and b"seq_first_block" in pkv.lib().pkv_last_error()
