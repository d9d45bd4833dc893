"""A continuous-batching decode step over device-resident block tables (binding layer).

Orders the library's calls for one serving step of a batch whose sequences may share
prefix blocks, and owns the buffers that stay alive between steps.  It holds no arithmetic
of the method: every step of it is a C ABI call.

One step ("What is PagedAttention?", glossary, "How It Works: Map Logical to Physical
Blocks" and "Share Without Mutating State"; "PagedAttention: Optimizing KV Cache in vLLM",
§4 "Copy-on-Write"):
  1. the host allocator appends one token to every sequence (pkv_seq_append), writing the
     slots and any copy-on-write pairs into one of two pinned host buffers;
  2. the copy-on-write pairs, when there are any, go to the device asynchronously and
     pkv_copy_blocks copies the shared partial tails;
  3. pkv_apply_append updates the device copies of the tables and lengths, reading the slots
     straight from the pinned buffer (no upload);
  4. pkv_paged_decode_step_split stores each sequence's new token into its slot and runs the
     split pass over every token, then pkv_paged_attention_reduce merges.  With prefix groups
     (``prefix_groups=True``), pkv_paged_decode_step_grouped does both passes instead, reading
     each group's shared blocks once for all its sequences; the groups (pkv_alloc_prefix_groups)
     are taken again after every append that copied a shared tail, and go to the device from
     the same pinned buffer.
The two host buffers alternate, so the host prepares step i+1 while the device runs step i.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import (BF16, F32, apply_append, copy_blocks, paged_attention_default_splits, paged_attention_grouped_workspace_size,
               paged_attention_reduce, paged_attention_workspace_size, paged_decode_step_grouped,
               paged_decode_step_split, set_launch_events, _dtype_code, _pool_dims)


class _HostBuf:
    def __init__(self, n: int):
        self.slots = torch.empty(n, dtype=torch.int64, pin_memory=True)
        self.cow = torch.empty((n, 2), dtype=torch.int32, pin_memory=True)
        self.groups = torch.empty((3, n), dtype=torch.int32, pin_memory=True)
        self.done = torch.cuda.Event()


class DecodeStep:
    """Decode steps for the sequences ``members`` of ``alloc`` over the pools ``k_cache`` /
    ``v_cache`` ([num_blocks, Hkv, bs * head_dim]).

    max_blocks: width of the device block tables (room for every block the steps will add).
    shared_prefix: read each sequence's shared leading blocks through the caches
    (``alloc.shared_prefix_blocks``, taken once here; later copy-on-write only shortens a
    shared prefix by its tail, and a stale count changes which loads are cached, never the
    result).  num_splits: as for the decode entry points (0 = the default count).
    """

    def __init__(self, alloc, members, k_cache, v_cache, head_dim: int, num_q_heads: int, max_blocks: int,
                 num_splits: int = 0, shared_prefix: bool = True, prefix_groups: bool = False):
        self.alloc = alloc
        self.members = np.ascontiguousarray(members, dtype=np.int64)
        self.k, self.v = k_cache, v_cache
        self.D = head_dim
        self.num_blocks, self.Hkv, self.bs = _pool_dims(k_cache, head_dim)
        dev = k_cache.device
        B = len(self.members)
        kd = _dtype_code(k_cache.dtype)
        qd = F32 if kd == F32 else BF16          # queries and new tokens: f32 for an f32 cache, else bf16
        self.num_splits = int(num_splits) or paged_attention_default_splits(head_dim, self.bs, qd, kd)
        tables, lens = alloc.block_tables(self.members, max_blocks)
        self.max_blocks = int(max_blocks)
        self.max_len = int(lens.max()) if B else 0   # every member grows by one token a step
        self.tables = torch.from_numpy(tables).to(dev)
        self.lens = torch.from_numpy(lens).to(dev)
        counts = alloc.shared_prefix_blocks(self.members)
        self.shared_counts = counts
        self.shared = torch.from_numpy(counts).to(dev) if shared_prefix and counts.any() else None
        self.prefix_groups = prefix_groups
        self.max_chunk = 32 // (num_q_heads // self.Hkv)
        if prefix_groups:
            self.shared = None                 # shared blocks are read once, streamed
            self.groups = torch.empty((3, B), dtype=torch.int32, device=dev)
            self._groups_host = None
            nbytes = paged_attention_grouped_workspace_size(B, num_q_heads, self.Hkv, head_dim, self.bs, qd, kd,
                                                            self.num_splits, max_blocks)
        else:
            nbytes = paged_attention_workspace_size(B, num_q_heads, self.Hkv, head_dim, self.bs, qd, kd,
                                                    self.num_splits)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.cow_d = torch.empty((B, 2), dtype=torch.int32, device=dev)
        self.bufs = [_HostBuf(B), _HostBuf(B)]
        self.steps = 0
        self.host_alloc_s = 0.0           # host time spent in the allocator's append
        self.last_slots = None
        self.last_cows = None

    def run(self, out, q, k_new, v_new, scale, k_scale=1.0, v_scale=1.0, kernel_events=None, after_upload=None):
        """Enqueues one step on the current stream; returns the number of copy-on-write pairs.

        kernel_events: an optional (start, stop) pair of recorded torch events that the split
        kernel's own dispatch records (set_launch_events).  after_upload: an optional event
        recorded once the pair upload is enqueued."""
        if -(-(self.max_len + 1) // self.bs) > self.max_blocks:
            # The device tables have no room for the new token's block: pkv_apply_append would
            # leave those rows unchanged, and the fused write would land on the old last token.
            raise ValueError(f"a sequence would grow past max_blocks={self.max_blocks} blocks of the device "
                             f"block tables ({self.max_len + 1} tokens)")
        hb = self.bufs[self.steps % 2]
        hb.done.synchronize()                 # the kernels that read this buffer have run
        self.steps += 1
        t0 = time.perf_counter()
        _, cows = self.alloc.append(self.members, hb.slots.numpy(), hb.cow.numpy())
        self.host_alloc_s += time.perf_counter() - t0
        self.max_len += 1
        n_cow = len(cows)
        self.last_slots = hb.slots.numpy().copy()
        self.last_cows = np.array(cows, dtype=np.int32).reshape(-1, 2)
        stream = torch.cuda.current_stream(self.k.device)
        if n_cow:
            self.cow_d[:n_cow].copy_(hb.cow[:n_cow], non_blocking=True)
        if after_upload is not None:
            after_upload.record(stream)
        if n_cow:
            copy_blocks(self.k, self.v, self.cow_d[:n_cow], self.D)
        apply_append(self.tables, self.lens, hb.slots, self.bs, self.num_blocks)
        if self.prefix_groups and (n_cow or self._groups_host is None):
            # A copy-on-write changed which leading blocks sequences share: take the groups again.
            t0 = time.perf_counter()
            self._groups_host = self.alloc.prefix_groups(self.members, self.max_chunk)
            self.host_alloc_s += time.perf_counter() - t0
            gh = hb.groups.numpy()
            for i in range(3):
                gh[i] = self._groups_host[i]
            self.groups.copy_(hb.groups, non_blocking=True)
        hb.done.record(stream)
        if kernel_events is not None:
            set_launch_events(kernel_events[0], kernel_events[1])
        if self.prefix_groups:
            paged_decode_step_grouped(out, q, k_new, v_new, self.k, self.v, self.tables, self.lens,
                                      (self.groups[0], self.groups[1], self.groups[2]), scale, k_scale, v_scale,
                                      num_splits=self.num_splits, workspace=self.ws)
            return n_cow
        paged_decode_step_split(out, q, k_new, v_new, self.k, self.v, self.tables, self.lens, scale, k_scale,
                                v_scale, num_splits=self.num_splits, workspace=self.ws,
                                shared_prefix_blocks=self.shared)
        paged_attention_reduce(out, q, self.k, self.v, self.tables, self.lens, scale, k_scale, v_scale,
                               num_splits=self.num_splits, workspace=self.ws, shared_prefix_blocks=self.shared)
        return n_cow
