"""Decode attention that allocates nothing (pkv_paged_attention_decode_noalloc) against the
entry point with a caller-given workspace, through the C ABI.

Two calls in a row, the second over a smaller batch, so the second runs over the first's
leftover scratch contents; each must give the same output bytes as pkv_paged_attention_decode
at the same split count (the same kernels), and both must match the fp64 oracle within the
bf16 tolerance |d| <= 2e-2 + 1e-2 |ref|.  Nothing in these calls allocates: the inputs are
made beforehand, and the call itself takes no workspace.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_329_amd as pkv
from oracle import attention as oatt
from synth import WORKLOADS, make_decode_case

from gpu_helpers import as_f64, assert_close, decode, log, pack, raw_bytes, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(case):
    wl = case.wl
    k, v = pack(case)
    q = to_dev(case.q, wl.q_dtype)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).cuda()
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    return k, v, q, tables, lens


def test_noalloc_decode_matches_the_workspace_entry_point():
    require_gpu()
    big = make_decode_case(WORKLOADS["llama3_8b_bf16"], 0)                       # the full 64-sequence batch
    small = make_decode_case(WORKLOADS["llama3_8b_bf16"].scaled(batch=5, length_dist=("uniform", 1, 700)), 1)
    prepared = [(c, _inputs(c)) for c in (big, small)]
    outs = [torch.empty_like(inp[2]) for _, inp in prepared]
    torch.cuda.synchronize()
    for (case, (k, v, q, tables, lens)), out in zip(prepared, outs):
        log(f"noalloc decode: batch {case.wl.batch}, sum L {int(case.lengths.sum())}")
        pkv.paged_attention_decode_noalloc(out, q, k, v, tables, lens, case.scale)
        torch.cuda.synchronize()
    for (case, (k, v, q, tables, lens)), out in zip(prepared, outs):
        want = decode(case, k, v)
        assert raw_bytes(out) == raw_bytes(want)
        seqs = list(range(case.wl.batch)) if case.wl.batch <= 8 else [0, 1, int(np.argmax(case.lengths))]
        assert_close(as_f64(out)[seqs], oatt.decode_case(case, seqs), case.wl.kv_dtype, "noalloc")


def test_noalloc_decode_fp8_and_explicit_splits():
    """An fp8 cache (4 workgroups per CU by default) and an explicit split count, again twice
    in a row with the smaller batch second."""
    require_gpu()
    big = make_decode_case(WORKLOADS["fp8_kv"].scaled(batch=16, length_dist=("uniform", 1, 3000)), 2)
    small = make_decode_case(WORKLOADS["fp8_kv"].scaled(batch=3, length_dist=("uniform", 1, 500)), 3)
    for case in (big, small):
        k, v, q, tables, lens = _inputs(case)
        for n in (0, 300):
            out = torch.empty_like(q)
            pkv.paged_attention_decode_noalloc(out, q, k, v, tables, lens, case.scale, float(case.k_scale),
                                               float(case.v_scale), num_splits=n)
            torch.cuda.synchronize()
            assert raw_bytes(out) == raw_bytes(decode(case, k, v, num_splits=n))
            assert_close(as_f64(out), oatt.decode_case(case), case.wl.kv_dtype, f"noalloc fp8 splits {n}")


def test_noalloc_decode_rejects_too_much_scratch():
    require_gpu()
    case = make_decode_case(WORKLOADS["llama3_8b_bf16"].scaled(batch=4, length_dist=("uniform", 1, 300)), 4)
    k, v, q, tables, lens = _inputs(case)
    out = torch.empty_like(q)
    with pytest.raises(pkv.PagedKVError, match="scratch"):
        pkv.paged_attention_decode_noalloc(out, q, k, v, tables, lens, case.scale, num_splits=200000)
