// Host block allocator: free list, per-block reference counts, sharing and
// copy-on-write decisions.  It only produces block tables, slots and copy lists; the
// device kernels consume them.
//
// Rules (pages cited by title and section):
//  * "What is PagedAttention?" (qubittool glossary), "How It Works: Map Logical to
//    Physical Blocks": a sequence's logical blocks map to arbitrary physical blocks; a
//    prefill takes enough blocks for its tokens; a decode step fills the partly used
//    last block and takes a new one only when it is full; an allocation that cannot be
//    met fails explicitly without touching other sequences — here every call is
//    all-or-nothing: it checks that the free list covers the whole request first.
//  * Same page, "Share Without Mutating State", and "PagedAttention: Optimizing KV
//    Cache in vLLM" (grasp.study), §4 "Advanced Benefit: Zero-Cost Sharing with
//    Copy-on-Write": shared blocks are immutable and reference counted; a write into a
//    block whose count exceeds one first takes a private block with a copy of it,
//    repoints only the writer's table entry and drops the old block's count; a block
//    whose count reaches zero returns to the free list.
//  * "What is PagedAttention?", "How It Works: Map Logical to Physical Blocks": an
//    allocation that cannot be met must lead to admission control, preemption, swap or
//    rejection.  pkv_seq_swap moves a sequence between two allocators (the device pool's
//    and a host pool's), returning the block copies the move needs.
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "status.h"

struct pkv_alloc {
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<uint32_t> refcount;
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t length = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

using pkv::fail;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t take_block(pkv_alloc* a) {
  int32_t b = a->free_stack.back();
  a->free_stack.pop_back();
  a->refcount[b] = 1;
  return b;
}

void release_block(pkv_alloc* a, int32_t b) {
  if (--a->refcount[b] == 0) a->free_stack.push_back(b);
}

// Appends one token to `s`; the caller has checked that the free list can cover it.
int64_t append_token(pkv_alloc* a, pkv_alloc::Seq& s, int32_t* cow_pair, int* n_cow) {
  const int bs = a->block_size;
  if (s.length % bs == 0) {
    s.blocks.push_back(take_block(a));
  } else {
    int32_t tail = s.blocks.back();
    if (a->refcount[tail] > 1) {
      int32_t fresh = take_block(a);
      a->refcount[tail] -= 1;  // still > 0: other sequences keep it
      s.blocks.back() = fresh;
      if (cow_pair) {
        cow_pair[2 * *n_cow + 0] = tail;
        cow_pair[2 * *n_cow + 1] = fresh;
      }
      ++*n_cow;
    }
  }
  int64_t pos = s.length++;
  return int64_t(s.blocks[pos / bs]) * bs + pos % bs;
}

}  // namespace

extern "C" {

pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PKV_INVALID_ARG, "pkv_alloc_create: num_blocks=%d block_size=%d must be positive",
         num_blocks, block_size);
    return nullptr;
  }
  auto* a = new (std::nothrow) pkv_alloc;
  if (!a) {
    fail(PKV_INVALID_ARG, "pkv_alloc_create: out of host memory");
    return nullptr;
  }
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        fail(PKV_INVALID_ARG, "pkv_alloc_create: free_order is not a permutation (entry %d = %d)",
             i, b);
        return nullptr;
      }
      seen[b] = 1;
      a->free_stack[num_blocks - 1 - i] = b;
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) a->free_stack[num_blocks - 1 - i] = i;
  }
  return a;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

pkv_status pkv_seq_create(pkv_alloc* a, int64_t seq_id, int64_t length, int64_t* slots_out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_create: null allocator");
  if (length < 0) return fail(PKV_INVALID_ARG, "pkv_seq_create: negative length %lld", (long long)length);
  if (a->seqs.count(seq_id))
    return fail(PKV_INVALID_ARG, "pkv_seq_create: sequence %lld already exists", (long long)seq_id);
  int64_t need = ceil_div(length, a->block_size);
  if (need > int64_t(a->free_stack.size()))
    return fail(PKV_OUT_OF_BLOCKS, "pkv_seq_create: needs %lld blocks, %zu free", (long long)need,
                a->free_stack.size());
  pkv_alloc::Seq s;
  s.blocks.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(take_block(a));
  s.length = length;
  if (slots_out)
    for (int64_t t = 0; t < length; ++t)
      slots_out[t] = int64_t(s.blocks[t / a->block_size]) * a->block_size + t % a->block_size;
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child, int64_t prefix_len) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_fork: null allocator");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end())
    return fail(PKV_UNKNOWN_SEQ, "pkv_seq_fork: unknown parent %lld", (long long)parent);
  if (a->seqs.count(child))
    return fail(PKV_INVALID_ARG, "pkv_seq_fork: child %lld already exists", (long long)child);
  if (prefix_len < 0 || prefix_len > it->second.length)
    return fail(PKV_INVALID_ARG, "pkv_seq_fork: prefix_len %lld outside [0, %lld]",
                (long long)prefix_len, (long long)it->second.length);
  pkv_alloc::Seq c;
  int64_t nb = ceil_div(prefix_len, a->block_size);
  c.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + nb);
  for (int32_t b : c.blocks) a->refcount[b] += 1;
  c.length = prefix_len;
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

pkv_status pkv_seq_extend(pkv_alloc* a, int64_t seq_id, int64_t n, int64_t* slots_out,
                          int32_t* cow_out, int* n_cow_out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_extend: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PKV_UNKNOWN_SEQ, "pkv_seq_extend: unknown sequence %lld", (long long)seq_id);
  if (n < 0) return fail(PKV_INVALID_ARG, "pkv_seq_extend: negative count %lld", (long long)n);
  pkv_alloc::Seq& s = it->second;
  const int bs = a->block_size;
  bool cow = n > 0 && s.length % bs != 0 && a->refcount[s.blocks.back()] > 1;
  int64_t need = (cow ? 1 : 0) + ceil_div(s.length + n, bs) - ceil_div(s.length, bs);
  if (need > int64_t(a->free_stack.size()))
    return fail(PKV_OUT_OF_BLOCKS, "pkv_seq_extend: needs %lld blocks, %zu free", (long long)need,
                a->free_stack.size());
  int n_cow = 0;
  for (int64_t i = 0; i < n; ++i) {
    int64_t slot = append_token(a, s, cow_out, &n_cow);
    if (slots_out) slots_out[i] = slot;
  }
  if (n_cow_out) *n_cow_out = n_cow;
  return PKV_OK;
}

pkv_status pkv_seq_append(pkv_alloc* a, const int64_t* seq_ids, int n, int64_t* slots_out,
                          int32_t* cow_out, int* n_cow_out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_append: null allocator");
  if (n < 0 || (n > 0 && (!seq_ids || !slots_out || !cow_out || !n_cow_out)))
    return fail(PKV_INVALID_ARG, "pkv_seq_append: n=%d with a null array", n);
  std::vector<pkv_alloc::Seq*> seqs(n);
  std::unordered_set<int64_t> distinct;
  for (int i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_UNKNOWN_SEQ, "pkv_seq_append: unknown sequence %lld", (long long)seq_ids[i]);
    if (!distinct.insert(seq_ids[i]).second)
      return fail(PKV_INVALID_ARG, "pkv_seq_append: sequence %lld listed twice",
                  (long long)seq_ids[i]);
    seqs[i] = &it->second;
  }
  // Count the blocks the step needs by replaying it on reference counts alone: a full
  // tail takes a new block; a shared partial tail takes a copy while its count (as
  // lowered by earlier copies in this call) exceeds one.
  const int bs = a->block_size;
  std::unordered_map<int32_t, uint32_t> sim;
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const pkv_alloc::Seq& s = *seqs[i];
    if (s.length % bs == 0) {
      ++need;
      continue;
    }
    int32_t tail = s.blocks.back();
    auto f = sim.find(tail);
    uint32_t rc = f == sim.end() ? a->refcount[tail] : f->second;
    if (rc > 1) {
      ++need;
      sim[tail] = rc - 1;
    }
  }
  if (need > int64_t(a->free_stack.size()))
    return fail(PKV_OUT_OF_BLOCKS, "pkv_seq_append: step needs %lld blocks, %zu free",
                (long long)need, a->free_stack.size());
  int n_cow = 0;
  for (int i = 0; i < n; ++i) slots_out[i] = append_token(a, *seqs[i], cow_out, &n_cow);
  *n_cow_out = n_cow;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_alloc* a, int64_t seq_id) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_free: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PKV_UNKNOWN_SEQ, "pkv_seq_free: unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.blocks) release_block(a, b);
  a->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_seq_swap(pkv_alloc* from, pkv_alloc* to, int64_t seq_id, int32_t* pairs_out,
                        int* n_pairs_out) {
  if (!from || !to || from == to)
    return fail(PKV_INVALID_ARG, "pkv_seq_swap: needs two distinct allocators");
  if (from->block_size != to->block_size)
    return fail(PKV_INVALID_ARG, "pkv_seq_swap: block sizes differ (%d, %d)", from->block_size,
                to->block_size);
  auto it = from->seqs.find(seq_id);
  if (it == from->seqs.end())
    return fail(PKV_UNKNOWN_SEQ, "pkv_seq_swap: unknown sequence %lld", (long long)seq_id);
  if (to->seqs.count(seq_id))
    return fail(PKV_INVALID_ARG, "pkv_seq_swap: sequence %lld already in the destination",
                (long long)seq_id);
  const size_t n = it->second.blocks.size();
  if (n > 0 && !pairs_out) return fail(PKV_INVALID_ARG, "pkv_seq_swap: null pairs_out");
  if (n > to->free_stack.size())
    return fail(PKV_OUT_OF_BLOCKS, "pkv_seq_swap: needs %zu blocks, %zu free in the destination", n,
                to->free_stack.size());
  // Every logical block gets a private destination block: sharing does not survive a swap.
  pkv_alloc::Seq moved;
  moved.length = it->second.length;
  moved.blocks.reserve(n);
  for (size_t j = 0; j < n; ++j) {
    const int32_t tb = take_block(to);
    pairs_out[2 * j + 0] = it->second.blocks[j];
    pairs_out[2 * j + 1] = tb;
    moved.blocks.push_back(tb);
  }
  for (int32_t b : it->second.blocks) release_block(from, b);
  from->seqs.erase(it);
  to->seqs.emplace(seq_id, std::move(moved));
  if (n_pairs_out) *n_pairs_out = int(n);
  return PKV_OK;
}

pkv_status pkv_alloc_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int n,
                                  int max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_alloc_block_tables: null allocator");
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || (!tables_out && max_blocks > 0))))
    return fail(PKV_INVALID_ARG, "pkv_alloc_block_tables: bad arguments");
  for (int i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_UNKNOWN_SEQ, "pkv_alloc_block_tables: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (int64_t(it->second.blocks.size()) > max_blocks)
      return fail(PKV_INVALID_ARG, "pkv_alloc_block_tables: sequence %lld has %zu blocks > %d",
                  (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
    if (it->second.length > INT32_MAX)
      return fail(PKV_INVALID_ARG, "pkv_alloc_block_tables: length does not fit int32");
  }
  for (int i = 0; i < n; ++i) {
    const auto& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + int64_t(i) * max_blocks;
    size_t nb = s.blocks.size();
    if (nb) std::memcpy(row, s.blocks.data(), nb * sizeof(int32_t));
    std::fill(row + nb, row + max_blocks, -1);
    if (lens_out) lens_out[i] = int32_t(s.length);
  }
  return PKV_OK;
}

pkv_status pkv_alloc_shared_prefix_blocks(const pkv_alloc* a, const int64_t* seq_ids, int n,
                                          int32_t* out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_alloc_shared_prefix_blocks: null allocator");
  if (n < 0 || (n > 0 && (!seq_ids || !out)))
    return fail(PKV_INVALID_ARG, "pkv_alloc_shared_prefix_blocks: bad arguments");
  for (int i = 0; i < n; ++i)
    if (a->seqs.find(seq_ids[i]) == a->seqs.end())
      return fail(PKV_UNKNOWN_SEQ, "pkv_alloc_shared_prefix_blocks: unknown sequence %lld",
                  (long long)seq_ids[i]);
  for (int i = 0; i < n; ++i) {
    const auto& blocks = a->seqs.find(seq_ids[i])->second.blocks;
    int32_t c = 0;
    while (size_t(c) < blocks.size() && a->refcount[blocks[c]] > 1) ++c;
    out[i] = c;
  }
  return PKV_OK;
}

pkv_status pkv_alloc_prefix_groups(const pkv_alloc* a, const int64_t* seq_ids, int n, int max_chunk,
                                   int32_t* chunk_first, int32_t* chunk_src, int32_t* group_blocks) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_alloc_prefix_groups: null allocator");
  if (n < 0 || max_chunk < 1 || (n > 0 && (!seq_ids || !chunk_first || !chunk_src || !group_blocks)))
    return fail(PKV_INVALID_ARG, "pkv_alloc_prefix_groups: bad arguments (n=%d max_chunk=%d)", n, max_chunk);
  std::vector<const pkv_alloc::Seq*> seq(n);
  for (int i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_UNKNOWN_SEQ, "pkv_alloc_prefix_groups: unknown sequence %lld", (long long)seq_ids[i]);
    seq[i] = &it->second;
  }
  auto first_shared = [&](int i) -> int32_t {
    const auto& b = seq[i]->blocks;
    return !b.empty() && a->refcount[b[0]] > 1 ? b[0] : -1;
  };
  auto shared_lead = [&](int i) {
    const auto& b = seq[i]->blocks;
    size_t c = 0;
    while (c < b.size() && a->refcount[b[c]] > 1) ++c;
    return c;
  };
  int i = 0;
  while (i < n) {
    // A group: the run of listed sequences starting with the same shared physical block.
    const int32_t head = first_shared(i);
    int end = i + 1;
    if (head >= 0)
      while (end < n && first_shared(end) == head) ++end;
    for (int c0 = i; c0 < end; c0 += max_chunk) {
      const int c1 = std::min(end, c0 + max_chunk);
      // The chunk reads its shared blocks from the member with the longest shared lead.
      int src = c0;
      for (int k = c0 + 1; k < c1; ++k)
        if (shared_lead(k) > shared_lead(src)) src = k;
      const auto& sb = seq[src]->blocks;
      int32_t most = 0;
      for (int k = c0; k < c1; ++k) {
        chunk_first[k] = c0;
        chunk_src[k] = src;
        if (k == src) continue;
        const auto& kb = seq[k]->blocks;
        int32_t same = 0;
        while (size_t(same) < kb.size() && size_t(same) < sb.size() && kb[same] == sb[same]) ++same;
        group_blocks[k] = same;
        most = std::max(most, same);
      }
      group_blocks[src] = most;
    }
    i = end;
  }
  return PKV_OK;
}

int pkv_alloc_num_free(const pkv_alloc* a) { return a ? int(a->free_stack.size()) : -1; }
int pkv_alloc_num_blocks(const pkv_alloc* a) { return a ? a->num_blocks : -1; }
int pkv_alloc_block_size(const pkv_alloc* a) { return a ? a->block_size : -1; }
int pkv_alloc_num_seqs(const pkv_alloc* a) { return a ? int(a->seqs.size()) : -1; }

int pkv_alloc_refcount(const pkv_alloc* a, int block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return int(a->refcount[block]);
}

pkv_status pkv_seq_info(const pkv_alloc* a, int64_t seq_id, int64_t* length_out,
                        int* num_blocks_out) {
  if (!a) return fail(PKV_INVALID_ARG, "pkv_seq_info: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PKV_UNKNOWN_SEQ, "pkv_seq_info: unknown sequence %lld", (long long)seq_id);
  if (length_out) *length_out = it->second.length;
  if (num_blocks_out) *num_blocks_out = int(it->second.blocks.size());
  return PKV_OK;
}

pkv_status pkv_alloc_stats_get(const pkv_alloc* a, pkv_alloc_stats* out) {
  if (!a || !out) return fail(PKV_INVALID_ARG, "pkv_alloc_stats_get: null argument");
  pkv_alloc_stats st{};
  st.num_blocks = a->num_blocks;
  st.free_blocks = int64_t(a->free_stack.size());
  st.num_seqs = int64_t(a->seqs.size());
  // Slots of each physical block that hold a token of at least one holder.
  std::vector<int32_t> filled(a->num_blocks, 0);
  const int bs = a->block_size;
  for (const auto& kv : a->seqs) {
    const pkv_alloc::Seq& q = kv.second;
    st.tokens += q.length;
    st.logical_blocks += int64_t(q.blocks.size());
    for (size_t j = 0; j < q.blocks.size(); ++j) {
      const int64_t in_block = std::min<int64_t>(bs, q.length - int64_t(j) * bs);
      filled[q.blocks[j]] = std::max<int32_t>(filled[q.blocks[j]], int32_t(in_block));
    }
  }
  for (int b = 0; b < a->num_blocks; ++b) {
    if (a->refcount[b] > 0) ++st.used_blocks;
    if (a->refcount[b] > 1) ++st.shared_blocks;
    st.stored_tokens += filled[b];
  }
  *out = st;
  return PKV_OK;
}

int pkv_alloc_free_list(const pkv_alloc* a, int32_t* ids_out, int cap) {
  if (!a) return -1;
  int n = int(a->free_stack.size());
  for (int i = 0; i < std::min(n, cap); ++i) ids_out[i] = a->free_stack[i];
  return n;
}

pkv_status pkv_build_slot_mapping(const int32_t* tables, const int32_t* lens, int num_seqs,
                                  int max_blocks, int block_size, int64_t* slots_out) {
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0 ||
      (num_seqs > 0 && (!tables || !lens || !slots_out)))
    return fail(PKV_INVALID_ARG, "pkv_build_slot_mapping: bad arguments");
  for (int s = 0; s < num_seqs; ++s)
    if (lens[s] < 0 || ceil_div(lens[s], block_size) > max_blocks)
      return fail(PKV_INVALID_ARG, "pkv_build_slot_mapping: sequence %d length %d exceeds its table",
                  s, lens[s]);
  int64_t n = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t* row = tables + int64_t(s) * max_blocks;
    for (int32_t t = 0; t < lens[s]; ++t)
      slots_out[n++] = int64_t(row[t / block_size]) * block_size + t % block_size;
  }
  return PKV_OK;
}

}  // extern "C"
