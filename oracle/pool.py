"""Physical KV block pool of the oracle (test infrastructure): write, copy, gather.

The pool is the project's own ABI (declared in include/pagedkv.h); this module
implements that declaration directly with numpy index arithmetic, independently of
the HIP code.  Terms:

* A K pool and a V pool, each ``num_blocks x Hkv`` regions of ``bs * D`` elements
  (element = float32 / bfloat16 / e4m3fn code), regions row-major over (block, head).
* A slot names one token position: ``slot = block * bs + offset`` (offset < bs).
  Appending a token writes its K and V into one slot ("What is PagedAttention?",
  qubittool glossary, "How It Works: Map Logical to Physical Blocks": decode fills the
  partly used last block and takes a new block only when that one is full).
* Inside a region, tokens come in sub-tiles of 16 (``bs / 16`` of them, 16*D elements
  each).  With ``x = 16 / element_bytes`` elements per 16-byte chunk:
    K element (t, d) of a sub-tile: ((d // x) * 16 + t) * x + d % x
    V element (t, d) of a sub-tile, x4 = x // 4:
        (((d // (4x)) * 4 + t // 4) * 16 + d % 16) * x + ((d // 16) % x4) * 4 + t % 4
  so a K chunk is x consecutive dims of one token, and a V chunk is 4 consecutive
  tokens for each of x4 dims that lie 16 apart.
* Copy-on-write copies a whole block (all heads, all bs slots) from a source to a
  destination block ("PagedAttention: Optimizing KV Cache in vLLM", grasp.study, §4
  "Advanced Benefit: Zero-Cost Sharing with Copy-on-Write": the writer gets a new block
  holding the shared block's contents and its own table entry is repointed).

Pinned by ``tests/test_oracle_pool.py``: offsets form a permutation of each region,
the chunk structure stated above, write-then-gather round trips, copy semantics.
"""
from __future__ import annotations

import numpy as np

from . import codecs

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}
STORE_DTYPE = {"f32": np.uint32, "bf16": np.uint16, "fp8_e4m3fn": np.uint8}


def k_offsets(bs: int, D: int, kv_dtype: str) -> np.ndarray:
    """[bs, D] element offset of K token ``o``, dim ``d`` inside a (block, head) region."""
    x = 16 // ELEM_BYTES[kv_dtype]
    o = np.arange(bs)[:, None]
    d = np.arange(D)[None, :]
    t = o % 16
    return (o // 16) * 16 * D + ((d // x) * 16 + t) * x + d % x


def v_offsets(bs: int, D: int, kv_dtype: str) -> np.ndarray:
    """[bs, D] element offset of V token ``o``, dim ``d`` inside a (block, head) region."""
    x = 16 // ELEM_BYTES[kv_dtype]
    x4 = x // 4
    o = np.arange(bs)[:, None]
    d = np.arange(D)[None, :]
    t = o % 16
    sub = (((d // (4 * x)) * 4 + t // 4) * 16 + d % 16) * x + ((d // 16) % x4) * 4 + t % 4
    return (o // 16) * 16 * D + sub


def empty_pool(num_blocks: int, Hkv: int, bs: int, D: int, kv_dtype: str, fill=0) -> np.ndarray:
    return np.full((num_blocks, Hkv, bs * D), fill, dtype=STORE_DTYPE[kv_dtype])


def _as_store(values: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "f32":
        return np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    return np.asarray(values, dtype=STORE_DTYPE[kv_dtype])


def encode_tokens(values: np.ndarray, in_dtype: str, kv_dtype: str, scale=1.0) -> np.ndarray:
    """New-token values -> the element bits the cache stores.

    f32 -> f32 and bf16 -> bf16 are bit copies; fp8 quantises float32 or bf16 inputs
    with the per-tensor inverse scale (``codecs.quantize_e4m3fn``).
    """
    if kv_dtype == "fp8_e4m3fn":
        inv = codecs.inverse_scale(scale)
        if in_dtype == "bf16":
            return codecs.quantize_bf16_to_e4m3fn(values, inv)
        return codecs.quantize_e4m3fn(np.asarray(values, dtype=np.float32), inv)
    if in_dtype != kv_dtype:
        raise ValueError(f"unsupported {in_dtype} -> {kv_dtype}")
    return _as_store(values, kv_dtype)


def write(pool_k, pool_v, new_k, new_v, slots, in_dtype, kv_dtype, bs, k_scale=1.0, v_scale=1.0):
    """Scatter tokens into the pools: token n goes to ``slots[n]``; negative slots are skipped.

    new_k / new_v: [T, Hkv, D] in ``in_dtype`` storage (float32 array or bf16 bits).
    """
    NB, Hkv, _ = pool_k.shape
    D = pool_k.shape[2] // bs
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    if not keep.any():
        return
    ek = encode_tokens(np.asarray(new_k)[keep], in_dtype, kv_dtype, k_scale)
    ev = encode_tokens(np.asarray(new_v)[keep], in_dtype, kv_dtype, v_scale)
    blk = slots[keep] // bs
    off = slots[keep] % bs
    ko = k_offsets(bs, D, kv_dtype)[off]          # [T', D]
    vo = v_offsets(bs, D, kv_dtype)[off]
    h = np.arange(Hkv)[None, :, None]
    pool_k[blk[:, None, None], h, ko[:, None, :]] = ek
    pool_v[blk[:, None, None], h, vo[:, None, :]] = ev


def copy_blocks(pool_k, pool_v, pairs):
    """pool[dst] = pool[src] for every (src, dst) pair, K and V, whole blocks."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        pool_k[dst] = pool_k[src]
        pool_v[dst] = pool_v[src]


def gather(pool, block_table_row, length: int, bs: int, D: int, kv_dtype: str, which: str):
    """Read one sequence's tokens back out of a pool in logical order -> [L, Hkv, D] bits."""
    offs = (k_offsets if which == "k" else v_offsets)(bs, D, kv_dtype)
    t = np.arange(length)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    o = offs[t % bs]                                   # [L, D]
    Hkv = pool.shape[1]
    h = np.arange(Hkv)[None, :, None]
    return pool[blk[:, None, None], h, o[:, None, :]]
