"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The allocation-free decode entry point exists for callers under graph capture, and the
other decode entry points take a caller-owned workspace, so all of them can be recorded
once and replayed.  No kernel of the library records a memset, and the split pass rewrites
its whole workspace record every launch, so every replay must give the eager result bit
for bit.  Each graph is replayed several times with eager work and synchronisations between
the replays; a fused decode step stores the same token into the same slot on every replay,
so it too repeats exactly.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_329_amd as pkv
from synth import WORKLOADS, make_decode_case

from gpu_helpers import pack, raw_bytes, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "llama3_8b_bf16": WORKLOADS["llama3_8b_bf16"].scaled(batch=6, length_dist=("uniform", 1, 700)),
    "fp8_kv": WORKLOADS["fp8_kv"].scaled(batch=4, length_dist=("uniform", 1, 1500)),
}


def _inputs(name):
    case = make_decode_case(CASES[name], 2)
    k, v = pack(case)
    wl = case.wl
    q = to_dev(case.q, wl.q_dtype)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).cuda()
    lens = torch.from_numpy(case.lengths.astype(np.int32)).cuda()
    return case, k, v, q, tables, lens


def _replays_equal(call, out, want, replays=4):
    """Capture call() once, then replay it `replays` times, clearing out and doing unrelated
    eager work before each replay; every replay must rewrite out with the eager bytes."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm-up outside the capture, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for r in range(replays):
        out.zero_()
        scratch.normal_()                        # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert raw_bytes(out) == want, f"replay {r}"


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_decode_replays_in_a_graph(name):
    require_gpu()
    case, k, v, q, tables, lens = _inputs(name)
    ks, vs = float(case.k_scale), float(case.v_scale)
    eager = torch.empty_like(q)
    pkv.paged_attention_decode_noalloc(eager, q, k, v, tables, lens, case.scale, ks, vs)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    _replays_equal(lambda: pkv.paged_attention_decode_noalloc(out, q, k, v, tables, lens, case.scale, ks, vs),
                   out, raw_bytes(eager))


@pytest.mark.parametrize("name", list(CASES))
def test_workspace_decode_and_decode_step_replay_in_a_graph(name):
    require_gpu()
    case, k, v, q, tables, lens = _inputs(name)
    wl = case.wl
    ks, vs = float(case.k_scale), float(case.v_scale)
    qd = pkv.BF16
    kd = pkv.FP8_E4M3FN if wl.kv_dtype == "fp8_e4m3fn" else pkv.BF16
    ws = torch.empty(pkv.paged_attention_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                        wl.block_size, qd, kd, 0),
                     dtype=torch.uint8, device="cuda")
    eager = torch.empty_like(q)
    pkv.paged_attention_decode(eager, q, k, v, tables, lens, case.scale, ks, vs, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    _replays_equal(lambda: pkv.paged_attention_decode(out, q, k, v, tables, lens, case.scale, ks, vs, workspace=ws),
                   out, raw_bytes(eager))

    # The fused decode step with each sequence's last token as the appended one: it stores
    # that token (already in the pool) again and attends over the same tokens.
    last = np.maximum(np.cumsum(case.lengths) - 1, 0)
    kn = to_dev(case.k[last], "bf16")
    vn = to_dev(case.v[last], "bf16")
    eager_step = torch.empty_like(q)
    pkv.paged_decode_step(eager_step, q, kn, vn, k, v, tables, lens, case.scale, ks, vs, workspace=ws)
    torch.cuda.synchronize()
    out_step = torch.empty_like(q)
    _replays_equal(lambda: pkv.paged_decode_step(out_step, q, kn, vn, k, v, tables, lens, case.scale, ks, vs,
                                                 workspace=ws),
                   out_step, raw_bytes(eager_step))
