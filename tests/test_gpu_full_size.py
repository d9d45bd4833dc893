"""Decode and multi-query parity at the full workload sizes, in the benchmark's launch
configuration.

The whole batch runs on the GPU with the default split count (one share per resident
wavefront slot, as the benchmark launches it); the fp64 oracle checks every sequence of the
batch, element by element (in chunks of sequences, to bound host memory).  Workloads:
  * Llama-3-8B-shaped bf16 layer: 64 sequences, 32 q / 8 kv heads, D 128, bs 16,
    lengths U{512..4096};
  * long-context split-K bf16: 8 sequences, 64 q / 8 kv heads, lengths U{32768..131072};
  * fp8 e4m3fn KV: 128 sequences, bs 32, lengths U{2048..16384}, per-tensor scales;
  * tiny fp32: 4 sequences, D 64, pool of 64 blocks (checked in full).
Multi-query workloads (the oracle checks sampled query rows: the first and last rows of the
longest and the shortest sequence, and 48 seeded picks):
  * causal prefill, bf16 and fp8 e4m3fn caches: 16 prompts of U{512..4096} tokens, every
    token a query (the query-tile path);
  * chunked prefill: the last 512 tokens of 16 contexts of U{1024..8192} tokens;
  * drafted-token checks: 64 sequences of U{512..4096} tokens, 5 queries each (the
    few-query split path).
"""
import numpy as np
import pytest

from oracle import attention as oatt
from synth import WORKLOADS, make_decode_case, make_prefill_case

from gpu_helpers import as_f64, assert_close, check_all_sequences, decode, log, pack, prefill, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b_bf16", "long_ctx_splitk_bf16", "fp8_kv"])
def test_full_size_parity(name):
    require_gpu()
    wl = WORKLOADS[name]
    case = make_decode_case(wl, 0)
    log(f"full size {name}: sum L = {int(case.lengths.sum())}, pool {case.num_blocks} blocks")
    k, v = pack(case)
    got = as_f64(decode(case, k, v))
    assert np.all(np.isfinite(got))
    check_all_sequences(got, case, name)


def _sample_rows(case, rng, extra=48):
    qs = np.asarray(case.query_start, dtype=np.int64)
    rows = set()
    for s in (int(np.argmin(case.lengths)), int(np.argmax(case.lengths))):
        if qs[s + 1] > qs[s]:
            rows.update((int(qs[s]), int(qs[s + 1]) - 1))
    rows.update(int(r) for r in rng.choice(int(qs[-1]), size=extra, replace=False))
    return sorted(rows)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["prefill_llama3_8b_bf16", "chunked_prefill_llama3_8b_bf16",
                                  "spec_verify_llama3_8b_bf16", "prefill_fp8_kv"])
def test_full_size_multi_query_parity(name):
    require_gpu()
    wl = WORKLOADS[name]
    case = make_prefill_case(wl, 0)
    log(f"full size {name}: {int(case.query_start[-1])} query rows, sum L = {int(case.lengths.sum())}, "
        f"pool {case.num_blocks} blocks")
    k, v = pack(case)
    got = as_f64(prefill(case, k, v))
    assert np.all(np.isfinite(got))
    rows = _sample_rows(case, np.random.default_rng(1))
    log(f"oracle on query rows {rows}")
    assert_close(got[rows], oatt.prefill_case(case, rows), wl.kv_dtype, name)
