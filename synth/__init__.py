"""Seeded synthetic inputs for paged decode attention.

This module draws the inputs that both the HIP path and the fp64 oracle consume:
context lengths, a random permutation of physical block IDs, the query tensor and
each sequence's *logical* (contiguous, token-major) K and V in their storage
dtype.  It holds none of the method's arithmetic: no attention, no paging
address arithmetic, no fp8 quantisation.  Values are drawn as float32 N(0, 1) and,
for bf16 storage, rounded to bfloat16 by torch's own cast.

Streams: ``numpy.random.SeedSequence(seed).spawn(6)`` in the fixed order
[lengths, permutation, q, K, V, extra]; K and V further spawn one sub-stream per
sequence so that any one sequence can be re-drawn alone and so that the draws can
run on a thread pool (numpy releases the GIL while filling arrays).

The five workloads are the ones the project measures and tests against:
a tiny fp32 case, a Llama-3-8B-shaped bf16 decode layer, a continuous-batching
step with prefix sharing, a long-context split-K case and an fp8-KV case.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "DecodeCase",
    "PrefixStepCase",
    "PrefillCase",
    "make_decode_case",
    "make_prefill_case",
    "query_lengths",
    "make_prefix_step_case",
    "draw_lengths",
    "bf16_bits_from_f32",
]


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic paged-decode workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str          # "f32" | "bf16"
    kv_dtype: str         # "f32" | "bf16" | "fp8_e4m3fn"
    length_dist: tuple    # ("uniform", lo, hi) inclusive | ("lognormal", median, sigma, cap)
    pool_blocks: int | None = None   # fixed pool size; None = ceil(1.1 * blocks in use)
    prefix_group: int = 0            # sequences per shared-prefix group (0 = no sharing)
    prefix_len: int = 0              # tokens in each group's shared prefix
    query_dist: tuple = ("one",)     # query tokens per sequence: ("one",) | ("all",) = every
                                     # token (a prefill) | ("fixed", n) = the last min(n, L)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **changes) -> "Workload":
        return dataclasses.replace(self, **changes)


WORKLOADS: dict[str, Workload] = {
    # 4 sequences, lengths U{1..100}, 8 q heads = 8 kv heads, D 64, bs 16, pool of 64 blocks.
    "tiny_fp32": Workload("tiny_fp32", 4, 8, 8, 64, 16, "f32", "f32", ("uniform", 1, 100), 64),
    # Llama-3-8B attention shape: 32 q heads / 8 kv heads, D 128, batch 64, lengths U{512..4096}.
    "llama3_8b_bf16": Workload("llama3_8b_bf16", 64, 32, 8, 128, 16, "bf16", "bf16",
                               ("uniform", 512, 4096)),
    # Continuous-batching step: 256 sequences in groups of 8 sharing a 1024-token prefix,
    # lengths lognormal (median 1000, sigma 1.0) capped at 8192.
    "cont_batch_prefix_bf16": Workload("cont_batch_prefix_bf16", 256, 32, 8, 128, 16, "bf16", "bf16",
                                       ("lognormal", 1000.0, 1.0, 8192), None, 8, 1024),
    # Long context: 8 sequences, 64 q heads / 8 kv heads, lengths U{32768..131072}.
    "long_ctx_splitk_bf16": Workload("long_ctx_splitk_bf16", 8, 64, 8, 128, 16, "bf16", "bf16",
                                     ("uniform", 32768, 131072)),
    # fp8 e4m3fn KV cache with per-tensor scales, bs 32, lengths U{2048..16384}.
    "fp8_kv": Workload("fp8_kv", 128, 32, 8, 128, 32, "bf16", "fp8_e4m3fn",
                       ("uniform", 2048, 16384)),
    # Several query tokens per sequence, causal over the same pool.
    # Small fp32 case with grouped heads, every token a query (a prefill).
    "prefill_tiny_fp32": Workload("prefill_tiny_fp32", 4, 8, 4, 64, 16, "f32", "f32",
                                  ("uniform", 1, 100), 64, query_dist=("all",)),
    # Llama-3-8B prefill: 16 prompts of U{512..4096} tokens.
    "prefill_llama3_8b_bf16": Workload("prefill_llama3_8b_bf16", 16, 32, 8, 128, 16, "bf16", "bf16",
                                       ("uniform", 512, 4096), query_dist=("all",)),
    # Chunked prefill: the last 512 tokens of contexts of U{1024..8192} tokens.
    "chunked_prefill_llama3_8b_bf16": Workload("chunked_prefill_llama3_8b_bf16", 16, 32, 8, 128, 16,
                                               "bf16", "bf16", ("uniform", 1024, 8192),
                                               query_dist=("fixed", 512)),
    # Speculative verification: 4 drafted tokens + 1 checked per sequence, decode-sized batch.
    "spec_verify_llama3_8b_bf16": Workload("spec_verify_llama3_8b_bf16", 64, 32, 8, 128, 16, "bf16",
                                           "bf16", ("uniform", 512, 4096), query_dist=("fixed", 5)),
    # Prefill over an fp8 e4m3fn cache (bs 32).
    "prefill_fp8_kv": Workload("prefill_fp8_kv", 16, 32, 8, 128, 32, "bf16", "fp8_e4m3fn",
                               ("uniform", 512, 4096), query_dist=("all",)),
}

_N_STREAMS = 6  # lengths, permutation, q, K, V, extra


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's cast and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def draw_lengths(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    dist = wl.length_dist
    if dist[0] == "uniform":
        _, lo, hi = dist
        return rng.integers(lo, hi + 1, size=wl.batch).astype(np.int64)
    if dist[0] == "lognormal":
        _, median, sigma, cap = dist
        z = rng.standard_normal(wl.batch)
        return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), 1, cap).astype(np.int64)
    raise ValueError(f"unknown length distribution {dist!r}")


def _draw_values(seed_seq: np.random.SeedSequence, shape, storage: str) -> np.ndarray:
    """N(0,1) float32 draws stored as f32, or bf16 bits for bf16 / fp8 storage.

    fp8 tensors are drawn as bf16 values; the quantiser of whichever side consumes them
    turns them into e4m3fn codes.
    """
    x = np.random.default_rng(seed_seq).standard_normal(shape, dtype=np.float32)
    if storage == "f32":
        return x
    return bf16_bits_from_f32(x)


def _draw_per_sequence(parent: np.random.SeedSequence, lengths, inner_shape, storage):
    """Concatenated [sum(L), *inner_shape] array, one sub-stream per sequence."""
    subs = parent.spawn(len(lengths))
    dtype = np.float32 if storage == "f32" else np.uint16
    offs = np.zeros(len(lengths) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    out = np.empty((int(offs[-1]),) + tuple(inner_shape), dtype=dtype)

    def fill(i):
        if lengths[i] > 0:
            out[offs[i]:offs[i + 1]] = _draw_values(subs[i], (int(lengths[i]),) + tuple(inner_shape), storage)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(lengths))))
    return out, offs


def _amax_scale(bits: np.ndarray) -> np.float32:
    """Per-tensor fp8 scale: largest |value| over the tensor divided by 448 (e4m3fn max).

    For finite bfloat16 values the magnitude order equals the integer order of the bits
    with the sign cleared, so the largest magnitude is found on the bits and only that
    one value is converted (by torch).
    """
    import torch

    if bits.size == 0:
        return np.float32(1.0)
    top = np.array([int(np.max(bits & np.uint16(0x7FFF)))], dtype=np.uint16)
    amax = np.float32(torch.from_numpy(top.view(np.int16)).view(torch.bfloat16).float().item())
    return np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)


@dataclass
class DecodeCase:
    """One batch of decode inputs with every sequence's K/V in logical order."""

    wl: Workload
    seed: int
    lengths: np.ndarray        # int64 [B]
    num_blocks: int            # physical pool size NB
    perm: np.ndarray           # int64 [NB]: perm[i] = physical block given out i-th
    block_tables: np.ndarray   # int32 [B, max_blocks], -1 past each sequence's blocks
    q: np.ndarray              # [B, Hq, D] float32 or bf16 bits (uint16)
    k: np.ndarray              # [sum L, Hkv, D] float32 or bf16 bits (fp8 storage: bf16 values)
    v: np.ndarray
    offsets: np.ndarray        # int64 [B+1] row offsets of each sequence in k / v
    k_scale: np.float32 = np.float32(1.0)
    v_scale: np.float32 = np.float32(1.0)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.wl.head_dim)

    def seq_k(self, s: int) -> np.ndarray:
        return self.k[self.offsets[s]:self.offsets[s + 1]]

    def seq_v(self, s: int) -> np.ndarray:
        return self.v[self.offsets[s]:self.offsets[s + 1]]


def _blocks_for(n_tokens: np.ndarray, bs: int) -> np.ndarray:
    # Number of fixed-size blocks that hold n tokens (the input recipe sizes the pool with it).
    return (n_tokens + bs - 1) // bs


def make_decode_case(wl: Workload, seed: int = 0, lengths=None) -> DecodeCase:
    """Draw a decode batch: lengths, a permuted physical pool, q and logical K/V.

    Physical blocks are handed out as ``perm[0], perm[1], ...`` in sequence-major,
    logical-ascending order, so consecutive logical blocks of a sequence land at
    unrelated physical positions.
    """
    ss = np.random.SeedSequence(seed).spawn(_N_STREAMS)
    if lengths is None:
        lengths = draw_lengths(wl, np.random.default_rng(ss[0]))
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.shape == (wl.batch,)
    bs = wl.block_size
    nb = _blocks_for(lengths, bs)
    used = int(nb.sum())
    num_blocks = wl.pool_blocks if wl.pool_blocks is not None else max(1, math.ceil(1.1 * used))
    if used > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {used} blocks")
    perm = np.random.default_rng(ss[1]).permutation(num_blocks).astype(np.int64)
    max_blocks = max(1, int(nb.max()) if len(nb) else 1)
    tables = np.full((wl.batch, max_blocks), -1, dtype=np.int32)
    pos = 0
    for s in range(wl.batch):
        tables[s, :nb[s]] = perm[pos:pos + nb[s]]
        pos += int(nb[s])
    q = _draw_values(ss[2], (wl.batch, wl.num_q_heads, wl.head_dim), wl.q_dtype)
    kv_store = "f32" if wl.kv_dtype == "f32" else "bf16"
    k, offs = _draw_per_sequence(ss[3], lengths, (wl.num_kv_heads, wl.head_dim), kv_store)
    v, _ = _draw_per_sequence(ss[4], lengths, (wl.num_kv_heads, wl.head_dim), kv_store)
    case = DecodeCase(wl, seed, lengths, num_blocks, perm, tables, q, k, v, offs)
    if wl.kv_dtype == "fp8_e4m3fn":
        case.k_scale = _amax_scale(k)
        case.v_scale = _amax_scale(v)
    return case


@dataclass
class PrefixStepCase:
    """Continuous-batching step over prefix-sharing groups.

    Group ``g`` owns a root prefix of ``prefix_len`` tokens.  Member ``i`` (in group
    ``i // prefix_group``) has ``lengths[i]`` cached tokens: the first
    ``min(lengths[i], prefix_len)`` are the root's, the rest are private.  The step
    appends one new token to every member and attends over ``lengths[i] + 1`` tokens.
    """

    wl: Workload
    seed: int
    lengths: np.ndarray         # int64 [B] cached tokens before the step
    num_blocks: int
    free_order: np.ndarray      # int32 [NB] order in which the allocator hands out blocks
    root_k: np.ndarray          # [groups, prefix_len, Hkv, D] bf16 bits
    root_v: np.ndarray
    priv_k: np.ndarray          # [sum max(0, L - prefix_len), Hkv, D]
    priv_v: np.ndarray
    priv_offsets: np.ndarray    # int64 [B+1]
    new_k: np.ndarray           # [B, Hkv, D] the token appended by the step
    new_v: np.ndarray
    q: np.ndarray               # [B, Hq, D]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.wl.head_dim)

    @property
    def groups(self) -> int:
        return self.wl.batch // self.wl.prefix_group

    def logical_kv(self, i: int):
        """Member i's K and V over all lengths[i] + 1 tokens after the step."""
        g = i // self.wl.prefix_group
        shared = min(int(self.lengths[i]), self.wl.prefix_len)
        a, b = self.priv_offsets[i], self.priv_offsets[i + 1]
        k = np.concatenate([self.root_k[g, :shared], self.priv_k[a:b], self.new_k[i:i + 1]])
        v = np.concatenate([self.root_v[g, :shared], self.priv_v[a:b], self.new_v[i:i + 1]])
        return k, v


def make_prefix_step_case(wl: Workload, seed: int = 0, lengths=None) -> PrefixStepCase:
    assert wl.prefix_group > 0 and wl.batch % wl.prefix_group == 0
    ss = np.random.SeedSequence(seed).spawn(_N_STREAMS)
    if lengths is None:
        lengths = draw_lengths(wl, np.random.default_rng(ss[0]))
    lengths = np.asarray(lengths, dtype=np.int64)
    groups = wl.batch // wl.prefix_group
    bs, P = wl.block_size, wl.prefix_len
    inner = (wl.num_kv_heads, wl.head_dim)
    # Pool: every root prefix plus, per member, enough blocks for all its tokens after the step
    # as if none were shared, plus 10%.
    bound = groups * int(_blocks_for(np.int64(P), bs)) + int(_blocks_for(lengths + 1, bs).sum())
    num_blocks = wl.pool_blocks if wl.pool_blocks is not None else math.ceil(1.1 * bound)
    free_order = np.random.default_rng(ss[1]).permutation(num_blocks).astype(np.int32)
    extra = ss[5].spawn(4)
    root_k = _draw_values(extra[0], (groups, P) + inner, "bf16")
    root_v = _draw_values(extra[1], (groups, P) + inner, "bf16")
    priv = np.maximum(lengths - P, 0)
    priv_k, poffs = _draw_per_sequence(ss[3], priv, inner, "bf16")
    priv_v, _ = _draw_per_sequence(ss[4], priv, inner, "bf16")
    new_k = _draw_values(extra[2], (wl.batch,) + inner, "bf16")
    new_v = _draw_values(extra[3], (wl.batch,) + inner, "bf16")
    q = _draw_values(ss[2], (wl.batch, wl.num_q_heads, wl.head_dim), wl.q_dtype)
    return PrefixStepCase(wl, seed, lengths, num_blocks, free_order, root_k, root_v,
                          priv_k, priv_v, poffs, new_k, new_v, q)


def query_lengths(wl: Workload, lengths: np.ndarray) -> np.ndarray:
    """Query tokens per sequence (the last n_s of its L_s tokens) under ``wl.query_dist``."""
    lengths = np.asarray(lengths, dtype=np.int64)
    kind = wl.query_dist[0]
    if kind == "one":
        return np.minimum(lengths, 1)
    if kind == "all":
        return lengths.copy()
    if kind == "fixed":
        return np.minimum(lengths, int(wl.query_dist[1]))
    raise ValueError(f"unknown query distribution {wl.query_dist!r}")


@dataclass
class PrefillCase(DecodeCase):
    """A batch whose sequences each have n_s query tokens: the last n_s of their L_s tokens.

    K / V hold every token, the queries' own included (a prefill writes them into the pool
    before attention reads them).  ``q`` is [sum n_s, Hq, D]; ``query_start`` is the int32
    prefix sum [B+1] of ``q_lens``.
    """

    q_lens: np.ndarray = None        # int64 [B]
    query_start: np.ndarray = None   # int32 [B+1]

    @property
    def num_q_tokens(self) -> int:
        return int(self.query_start[-1])


def make_prefill_case(wl: Workload, seed: int = 0, lengths=None, q_lens=None) -> PrefillCase:
    """Draw a multi-query batch: the decode case's lengths, pool and K/V, and a query
    tensor of sum n_s rows drawn from the extra stream."""
    base = make_decode_case(wl, seed, lengths)
    q_lens = query_lengths(wl, base.lengths) if q_lens is None else np.asarray(q_lens, dtype=np.int64)
    assert q_lens.shape == (wl.batch,) and np.all(q_lens >= 0)
    qs = np.zeros(wl.batch + 1, dtype=np.int32)
    qs[1:] = np.cumsum(q_lens)
    extra = np.random.SeedSequence(seed).spawn(_N_STREAMS)[5]
    q = _draw_values(extra.spawn(1)[0], (int(qs[-1]), wl.num_q_heads, wl.head_dim), wl.q_dtype)
    fields = {f.name: getattr(base, f.name) for f in dataclasses.fields(DecodeCase)}
    fields["q"] = q
    return PrefillCase(**fields, q_lens=q_lens, query_start=qs)
