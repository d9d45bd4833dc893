"""The KV pool in contiguous virtual memory mapped on demand (pkv_vmm_*), on the GPU.

Sequences' K/V written into per-sequence contiguous slices are read three ways: by the paged
decode kernel and the multi-query kernel through block tables that count up from each
slice's first block, and by the contiguous decode kernel, which computes block addresses
from the first block alone.  Each result is checked against the fp64 oracle (the pages fix
the result as attention over contiguous K/V: "PagedAttention: Optimizing KV Cache in vLLM",
§3), and each also gives the same bytes as the paged kernels over the same K/V scattered in
an ordinary pool (placement does not enter the arithmetic).  The mapped bytes follow the
page arithmetic and drop back when sequences are released.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_329_amd as pkv
from oracle import attention as oatt
from synth import WORKLOADS, make_prefill_case

from gpu_helpers import as_f64, assert_close, log, pack, prefill, raw_bytes, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _vmm_case(wl, seed, page_bytes=0):
    case = make_prefill_case(wl, seed)
    Hkv, D, bs = wl.num_kv_heads, wl.head_dim, wl.block_size
    nbs = [(int(L) + bs - 1) // bs for L in case.lengths]
    max_blocks = max(1, max(nbs))
    try:
        vmm = pkv.VmmPool(wl.batch, max_blocks, Hkv, bs, D, torch.bfloat16, page_bytes=page_bytes)
    except pkv.PagedKVError as e:
        pytest.skip(f"no virtual memory management here: {e}")
    tables = np.full((wl.batch, max_blocks), -1, dtype=np.int32)
    for s, nb in enumerate(nbs):
        vmm.reserve(s, nb)
        assert vmm.mapped_blocks(s) >= nb
        tables[s, :nb] = vmm.first_block(s) + np.arange(nb)
    slots = pkv.build_slot_mapping(tables, case.lengths.astype(np.int32), bs)
    pkv.kv_cache_write(to_dev(case.k, "bf16"), to_dev(case.v, "bf16"), vmm.k, vmm.v, torch.from_numpy(slots).cuda())
    return case, vmm, tables, nbs


@pytest.mark.parametrize("seed", [3, 4])
def test_vmm_pool_matches_the_oracle(seed):
    require_gpu()
    wl = WORKLOADS["chunked_prefill_llama3_8b_bf16"].scaled(batch=5, length_dist=("uniform", 1, 900),
                                                            query_dist=("fixed", 9))
    case, vmm, tables, nbs = _vmm_case(wl, seed)
    log(f"vmm granule {vmm.page_bytes} block {vmm.block_bytes} lengths {case.lengths.tolist()}")
    k, v = pack(case)
    # Decode: the last query row of each sequence attends to all of its tokens, which is the
    # oracle's causal query at position L - 1.
    last = case.query_start[1:] - 1
    ref_dec = oatt.prefill_case(case, last)
    q = to_dev(case.q[last], "bf16")
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    outs = {}
    for name, kk, vv, t in (("paged pool", k, v, case.block_tables), ("vmm slices", vmm.k, vmm.v, tables)):
        o = torch.empty_like(q)
        pkv.paged_attention_decode(o, q, kk, vv, torch.from_numpy(np.ascontiguousarray(t)).cuda(), lens, case.scale)
        torch.cuda.synchronize()
        assert_close(as_f64(o), ref_dec, "bf16", f"decode over the {name}")
        outs[name] = raw_bytes(o)
    assert outs["paged pool"] == outs["vmm slices"]
    # The contiguous kernel: block addresses from each slice's first block, no table.
    first = torch.tensor([vmm.first_block(s) for s in range(wl.batch)], dtype=torch.int32, device="cuda")
    oc = torch.empty_like(q)
    pkv.contiguous_attention_decode(oc, q, vmm.k, vmm.v, first, lens, tables.shape[1], case.scale)
    torch.cuda.synchronize()
    assert_close(as_f64(oc), ref_dec, "bf16", "contiguous decode over the vmm slices")
    assert raw_bytes(oc) == outs["paged pool"]
    # Multi-query attention over the slices.
    got = prefill(case, vmm.k, vmm.v, tables=tables)
    assert_close(as_f64(got), oatt.prefill_case(case), "bf16", "multi-query over the vmm slices")
    assert raw_bytes(got) == raw_bytes(prefill(case, k, v))
    vmm.close()


@pytest.mark.parametrize("page_bytes", [0, 65536])
def test_vmm_mapped_bytes_follow_pages_and_release(page_bytes):
    require_gpu()
    wl = WORKLOADS["llama3_8b_bf16"].scaled(batch=4, length_dist=("uniform", 1, 3000))
    case, vmm, tables, nbs = _vmm_case(wl, 5, page_bytes)
    g, bb = vmm.page_bytes, vmm.block_bytes
    per_seq = [-(-nb * bb // g) * g for nb in nbs]
    assert vmm.mapped_bytes == 2 * (g + sum(per_seq))
    vmm.release(1)
    assert vmm.mapped_bytes == 2 * (g + sum(per_seq) - per_seq[1]) and vmm.mapped_blocks(1) == 0
    vmm.reserve(1, nbs[1])
    assert vmm.mapped_bytes == 2 * (g + sum(per_seq))
    with pytest.raises(pkv.PagedKVError):
        vmm.reserve(1, 10 ** 6)            # beyond the sequence's slice
    vmm.close()


def test_vmm_release_waits_for_work_in_flight():
    """Releasing a slice right after enqueuing a decode that reads it is safe: the release
    waits for the device before unmapping, and the decode's output is the oracle's."""
    require_gpu()
    wl = WORKLOADS["llama3_8b_bf16"].scaled(batch=3, length_dist=("uniform", 200, 2000))
    case, vmm, tables, nbs = _vmm_case(wl, 6)
    last = case.query_start[1:] - 1
    q = to_dev(case.q[last], "bf16")
    o = torch.empty_like(q)
    pkv.paged_attention_decode(o, q, vmm.k, vmm.v, torch.from_numpy(np.ascontiguousarray(tables)).cuda(),
                               torch.from_numpy(case.lengths.astype(np.int32)).cuda(), case.scale)
    for s in range(wl.batch):
        vmm.release(s)
    torch.cuda.synchronize()
    assert_close(as_f64(o), oatt.prefill_case(case, last), "bf16", "decode enqueued before release")
    assert vmm.mapped_bytes == 2 * vmm.page_bytes
    vmm.close()
