// Paged decode attention for gfx950 (MI355X): split pass + merge pass.
//
// What is computed ("PagedAttention: Optimizing KV Cache in vLLM", grasp.study, §3
// "Making it Work: The PagedAttention Kernel"): the kernel looks up each request's
// block table, visits the physical blocks in logical order and folds them into a
// running softmax, which yields exactly attention over a contiguous K/V layout.
//
// How it maps onto CDNA4
//  * Work: the total work is the list of (sequence, kv-head group, block) triples in
//    sequence-major order, where a group is `coop` adjacent kv heads (4 when Hkv allows,
//    else 2 or 1); it is cut into splits / coop equal shares, one per group of `coop`
//    consecutive waves of a workgroup, so a wave's cost does not depend on how skewed the
//    context lengths are.  The waves of a group walk the same blocks side by side, each on
//    its own kv head, so together they stream the adjacent head regions of every block
//    (16 KiB of K, then of V, for bf16 D 128).  A share may end inside a (sequence, group)
//    unit; such a unit leaves one partial (max, sum, accumulator) per share and kv head,
//    and the merge pass combines them with the same rescaling the running softmax uses.
//    Units that fit in one share are finished in the split pass.
//  * Operands: a 16-token sub-tile of a (block, kv head) is one contiguous region; wave
//    load i, lane l reads the 16-byte chunk 64*i + l.  The pool layout makes that chunk
//    exactly lane l's operand of the gfx950 matrix instructions:
//      QK:  S^T[16 tokens][16 heads] = K[16 x D] . Q^T[D x 16] (heads >= G are zero),
//           A = K chunk (token l%16, dims of chunk 4i + l/16), B = the matching q dims.
//      PV:  O^T[16 dims][16 heads] += V^T[16 x 16 tokens] . P^T[16 tokens x 16 heads],
//           A = V chunk (4 tokens 4(l/16).. for dim l%16), B = the probabilities that
//           lane l already holds from QK (C layout: token 4(l/16)+j, head l%16).
//    So the softmax needs no data movement between the two products, and the per-head
//    statistics live in the lanes of head l%16.  No LDS is used: every K/V byte is
//    read by exactly one wave, straight into registers.
//  * Loads: K/V chunks carry the non-temporal hint, except in the leading blocks of a
//    sequence that the caller marks as shared with other sequences of the call (forked
//    prefixes); those go through ordinary cached loads, so that the sequences reading a
//    shared block at about the same time find it in L2 or the MALL.
//  * Running softmax (base 2): m = max(m, chunk max); rescale acc and sum by 2^(m_old-m);
//    p = 2^(s - m).  The chunk max needs two cross-row shuffles (xor 16, xor 32).
//  * Masking: tokens at or past the context length get s = -inf (select, so garbage or
//    NaN in unused slots cannot leak), and their V elements are zeroed before the PV
//    product.
//  * Types: (q, kv) = (f32, f32) uses v_mfma_f32_16x16x4_f32; (bf16, bf16) uses
//    v_mfma_f32_16x16x32_bf16 for QK and v_mfma_f32_16x16x16_bf16 for PV with p rounded
//    to bf16; (bf16, e4m3fn) widens each fp8 pair to bf16 with
//    v_cvt_scalef32_pk_bf16_fp8 (exact: every e4m3fn value is a bf16 value) and folds
//    k_scale into the logit scale and v_scale into the final normalisation.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <unordered_map>

#include "attention_tile.h"
#include "kv_codec.h"
#include "status.h"

namespace {

using namespace pkv::tile;

constexpr int kWavesPerWG = 4;
constexpr int kXcds = 8;   // MI355X: workgroups are dealt to the 8 XCDs round-robin
constexpr int kMaxGroup = 16;
constexpr int kGroupCols = 32;   // (member, query head) columns of a group share: two 16-column tiles
// Batches of up to kScanSeqs sequences: each workgroup of the prefix-group split pass scans
// both work lists into LDS, kScanSeqs / (kWavesPerWG * 64) sequences per thread.
constexpr int kScanSeqs = 512;
constexpr int kScanPerThread = kScanSeqs / (kWavesPerWG * 64);
// LDS entry of a sequence's group columns in the prefix-group pass: (group blocks << 10) |
// chunk first (kNoChunk when outside [0, num_seqs)); used while the table width is below
// 2^21 blocks.
constexpr int kNoChunk = 1023;
constexpr int kGlimMaxBlocks = 1 << 21;

// Work lists are cut by estimated cost, not by block count.  A unit (one sequence's blocks for
// one head group) weighs kUnitW plus kBlockW per block: its q and table round trip and its
// epilogue cost about 1.5 blocks' time, measured on MI355X (with equal blocks per share, a
// share crossing 16 units ended 54 us after one crossing a single unit, 1.5 blocks' time per
// extra unit).  A group share's block, with 32 columns of matrix and softmax work, weighs
// kGroupBlockW (measured 2.73 against 2.41 us per block).  A block belongs to the share
// holding its first weighted position.
constexpr int kBlockW = 8;
constexpr int kGroupBlockW = 9;
constexpr int kUnitW = 12;

__host__ __device__ __forceinline__ int unit_span(int nb, int block_w) { return nb > 0 ? nb * block_w + kUnitW : 0; }

// Shares of a work list of W weighted positions: at most `want`, and none shorter than a
// block's weight, so that every share lying inside a unit holds a block of it (the merge
// takes a piece from each share between the unit's first block and its last).
__host__ __device__ __forceinline__ int list_shares(int want, int W, int block_w) {
  return std::min(want, W / block_w);
}

// Blocks [j0, j1) of a unit (first weighted position unit_off, nb blocks of weight block_w)
// whose first weighted positions lie in [lo, hi).
__device__ __forceinline__ void unit_blocks_in(int unit_off, int nb, int block_w, int lo, int hi, int& j0, int& j1) {
  const int base = unit_off + kUnitW;
  j0 = lo <= base ? 0 : std::min(nb, (lo - base + block_w - 1) / block_w);
  j1 = hi <= base ? 0 : std::min(nb, (hi - base + block_w - 1) / block_w);
}

// Workspace layout: header (per-sequence work offsets and the split pass's record), partial
// accumulators, partial (max, sum) pairs; each part rounded up to 256 bytes.
__host__ __device__ constexpr int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }
__host__ __device__ constexpr int64_t header_bytes(int B) { return round256((int64_t(B) + 4) * 4); }
__host__ __device__ constexpr int64_t acc_bytes(int splits, int G, int D) {
  return round256(int64_t(splits) * 2 * G * D * 4);
}
__host__ __device__ constexpr int64_t ml_bytes(int splits, int G) { return round256(int64_t(splits) * 2 * G * 2 * 4); }

struct DecodeArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Workspace: a header at its start, then the partials.  The header is
  //   ws_seq[0..B-1]  work offset of sequence s (head groups * blocks of the sequences before it)
  //   ws_seq[B]       total work W
  //   ws_seq[B+1..3]  the split pass's share count, head-group width and num_seqs,
  // written by the split pass; the merge takes the layout of the partials from it, so it
  // always reads them where the split pass that preceded it wrote them.
  int* ws_seq;
  float* ws_acc;  // [splits*2][G][D]
  float* ws_ml;   // [splits*2][G][2]  (max in log2 units, sum)
  int64_t ws_bytes;
  int B, Hkv, G, num_blocks, max_blocks, splits;
  // Waves that walk one share together, each on its own kv head of the same blocks: the
  // work list is (sequence, group of `coop` kv heads, block).  A power of two that divides
  // both Hkv and kWavesPerWG, so a group's waves are consecutive waves of one workgroup.
  int coop;
  float qk_scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
  // Decode step with append: each sequence's token at position L-1 is taken from
  // k_new / v_new ([B][Hkv][D], q's dtype) and stored into its slot.
  const void* k_new;
  const void* v_new;
  uint8_t* k_cache_w;
  uint8_t* v_cache_w;
  float k_inv, v_inv;  // float32 1/k_scale, 1/v_scale (fp8 caches)
  // [B] or null: leading logical blocks of sequence s that other sequences also read.
  const int32_t* shared_prefix;
  // Contiguous placement (no block table): logical block j of sequence s is pool block
  // seq_first_block[s] + j.
  const int32_t* seq_first_block;
  // Prefix groups ([B] each, or null): the first sequence of s's column chunk, the chunk's
  // table source (read at the chunk's first sequence) and s's leading blocks that the group
  // pass reads for it (the same physical blocks as the source's first ones).
  const int32_t* chunk_first;
  const int32_t* chunk_src;
  const int32_t* group_blocks;
  // Grouped workspace parts (see grouped_layout): member pieces of units finished inside one
  // share, group pieces of shares, group pieces of units finished inside one share.
  float* ws_macc;  // [B * Hkv][G][D]
  float* ws_mml;   // [B * Hkv][G][2]
  float* ws_gacc;  // [splits * 2][kGroupCols][D]
  float* ws_gml;   // [splits * 2][kGroupCols][2]
  float* ws_fgacc; // [B * Hkv][kGroupCols][D]
  float* ws_fgml;  // [B * Hkv][kGroupCols][2]
  // [B][8] int32, when the split pass scans the lists in LDS (B <= kScanSeqs): sequence s's
  // member offset, its chunk's group offset, the chunk's blocks, s's group blocks, s's member
  // blocks and its chunk's first sequence, for the merge.
  int* ws_rec;
  int appending;   // 1 for the decode step with append (token L-1 is the appended one)
};


// Blocks holding a sequence's tokens (length clamped to what its table row can hold).
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int s, int bs) {
  int L = a.context_lens[s];
  L = L < 0 ? 0 : L;
  const int64_t cap = int64_t(a.max_blocks) * bs;
  if (L > cap) L = int(cap);
  return (L + bs - 1) / bs;
}

__device__ __forceinline__ int seq_len(const DecodeArgs& a, int s, int bs) {
  int L = a.context_lens[s];
  L = L < 0 ? 0 : L;
  const int64_t cap = int64_t(a.max_blocks) * bs;
  return L > cap ? int(cap) : L;
}

// Units (groups of `coop` kv heads) per sequence.
__device__ __forceinline__ int head_groups(const DecodeArgs& a) { return a.Hkv / a.coop; }

// Full blocks of sequence s's cached tokens (with append, token L-1 is not cached yet).
__device__ __forceinline__ int cached_full_blocks(const DecodeArgs& a, int s, int bs) {
  const int L = seq_len(a, s, bs);
  return (L - (a.appending && L > 0 ? 1 : 0)) / bs;
}

// Blocks the group pass reads for the chunk whose first sequence is f (0 unless f starts a
// well-formed chunk): the source's count, limited to the source's full cached blocks.
__device__ __forceinline__ int chunk_blocks(const DecodeArgs& a, int f, int bs) {
  const int M = kGroupCols / a.G;
  if (a.chunk_first[f] != f) return 0;
  const int src = a.chunk_src[f];
  if (src < f || src - f >= M || src >= a.B || a.chunk_first[src] != f) return 0;
  return min(max(a.group_blocks[src], 0), cached_full_blocks(a, src, bs));
}

// Leading blocks of sequence s that the group pass reads for it (its own count, limited to
// its full cached blocks and to its chunk's blocks; 0 when its chunk is not well formed).  The
// block receiving an appended token is never among them, so the appended token always falls
// in the sequence's own part.
__device__ __forceinline__ int group_skip(const DecodeArgs& a, int s, int bs) {
  const int M = kGroupCols / a.G;
  const int f = a.chunk_first[s];
  if (f < 0 || f > s || s - f >= M) return 0;
  return min(min(max(a.group_blocks[s], 0), chunk_blocks(a, f, bs)), cached_full_blocks(a, s, bs));
}

// Blocks of sequence s walked by the per-sequence (member) part: all of them, or with prefix
// groups those after the leading blocks the group pass reads.
template <bool GROUPED>
__device__ __forceinline__ int unit_blocks(const DecodeArgs& a, int s, int bs) {
  const int nb = seq_blocks(a, s, bs);
  if constexpr (GROUPED) return nb - group_skip(a, s, bs);
  return nb;
}

// Total work W = head_groups * sum_s unit_span(blocks(s)) (wave-uniform; the host checks it
// fits in int).
template <bool GROUPED = false>
__device__ int total_work(const DecodeArgs& a, int bs, int lane) {
  int acc = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int s = base + lane;
    acc += s < a.B ? unit_span(unit_blocks<GROUPED>(a, s, bs), kBlockW) : 0;
  }
  return wave_sum(acc) * head_groups(a);
}

// Group work: head_groups * sum over chunk first sequences f of their units' spans.
__device__ int group_work(const DecodeArgs& a, int bs, int lane) {
  int acc = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int s = base + lane;
    acc += s < a.B ? unit_span(chunk_blocks(a, s, bs), kGroupBlockW) : 0;
  }
  return wave_sum(acc) * head_groups(a);
}

// Per-unit spans of sequence s in the member list (unit_blocks<true>) and of the chunk that s
// starts in the group list (chunk_blocks), from the same definitions, with every lookup
// issued unconditionally (indices clamped into range, results selected): the sequence's own
// entries, then its chunk's, then the chunk sources', three dependent round trips in all.
struct SeqSpans {
  int mspan, gspan;   // per-unit spans in the member and group lists
  int skip;           // leading blocks the group pass reads for s (group_skip)
  int f, P;           // s's chunk (its first sequence) and that chunk's blocks, when skip > 0
  int L;              // s's clamped length
  int cf;             // chunk_first[s] as stored
};

__device__ __forceinline__ SeqSpans seq_spans(const DecodeArgs& a, int s, int bs) {
  const int M = kGroupCols / a.G;
  const int Ls = seq_len(a, s, bs);
  const int fs = a.chunk_first[s], gbs = a.group_blocks[s], srcs = a.chunk_src[s];
  const bool f_ok = fs >= 0 && fs <= s && s - fs < M;
  const int fc = f_ok ? fs : s;
  const int cf_f = a.chunk_first[fc], src_f = a.chunk_src[fc];
  const int sf = unsigned(src_f) < unsigned(a.B) ? src_f : 0;
  const int ss = unsigned(srcs) < unsigned(a.B) ? srcs : 0;
  const int cf_sf = a.chunk_first[sf], gb_sf = a.group_blocks[sf], L_sf = seq_len(a, sf, bs);
  const int cf_ss = a.chunk_first[ss], gb_ss = a.group_blocks[ss], L_ss = seq_len(a, ss, bs);
  auto full_blocks = [&](int L) { return (L - (a.appending && L > 0 ? 1 : 0)) / bs; };
  const bool ok_f = cf_f == fc && src_f >= fc && src_f - fc < M && src_f < a.B && cf_sf == fc;
  const int cb_f = ok_f ? min(max(gb_sf, 0), full_blocks(L_sf)) : 0;
  const int skip = f_ok ? min(min(max(gbs, 0), cb_f), full_blocks(Ls)) : 0;
  const bool ok_s = fs == s && srcs >= s && srcs - s < M && srcs < a.B && cf_ss == s;
  const int cb_s = ok_s ? min(max(gb_ss, 0), full_blocks(L_ss)) : 0;
  return SeqSpans{unit_span((Ls + bs - 1) / bs - skip, kBlockW), unit_span(cb_s, kGroupBlockW), skip, fc, cb_f, Ls, fs};
}

// Sequence whose units contain work position x (0 <= x < W), and the weighted positions of
// the units before it.  GROUP: over the group work list (chunk first sequences and their
// blocks).
template <bool GROUPED = false, bool GROUP = false>
__device__ void locate(const DecodeArgs& a, int bs, int lane, int x, int& s_out, int& off_out) {
  int base = 0;
  const int hg = head_groups(a);
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int s = b0 + lane;
    const int w = s < a.B ? (GROUP ? unit_span(chunk_blocks(a, s, bs), kGroupBlockW)
                                   : unit_span(unit_blocks<GROUPED>(a, s, bs), kBlockW)) * hg
                          : 0;
    const int incl = wave_incl_scan(w, lane);
    const int lo = base + (incl - w), hi = base + incl;
    const uint64_t hit = __ballot(w > 0 && lo <= x && x < hi);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      s_out = b0 + l;
      off_out = base + __builtin_amdgcn_readlane(incl - w, l);
      return;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  s_out = a.B;
  off_out = base;
}


// Element bits the cache stores for input element bits x (q's dtype) of k_new / v_new: f32
// and bf16 are stored as given; fp8 stores RNE(clamp(x * inv)), as the KV-cache write does.
template <int KV>
__device__ __forceinline__ uint32_t cache_bits(uint32_t x, float inv) {
  if constexpr (KV == PKV_FP8_E4M3FN) return pkv::e4m3fn_from_f32(pkv::bf16_bits_to_f32(x) * inv);
  return x;
}

// The value attention uses for cached element bits c (per-tensor scales applied outside).
template <int KV>
__device__ __forceinline__ float cache_value(uint32_t c) {
  if constexpr (KV == PKV_F32) return __uint_as_float(c);
  else if constexpr (KV == PKV_BF16) return pkv::bf16_bits_to_f32(c);
  else return e4m3fn_value(c);
}

// Input element e (q's dtype: 4 or 2 bytes) of a run of 16-byte words.
template <int QB>
__device__ __forceinline__ uint32_t input_element(const uint4* w, int e) {
  const uint4 c = w[(e * QB) / 16];
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
  const int k = e % (16 / QB);
  if constexpr (QB == 4) return d[k];
  else return (d[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

// The appended token of one unit, as this lane needs it, loaded when the segment that ends
// the unit starts (so that neither the fold nor the stores wait for memory):
//  k[i*QCH ..]: k_new dims X*(4i + lane/16) .. +X (the dims of this lane's q fragments,
//               and of its K chunk of load i),
//  vf[n][..]:   v_new dims 16n + 4*(lane/16) .. +3 (this lane's accumulator dims),
//  vs[i][e]:    v_new dim i*4X + 16e + lane%16 (its element of the V chunk of load i).
template <int KV, int D>
struct AppendRegs {
  static constexpr int QB = KvTraits<KV>::QB;
  static constexpr int X = 16 / KvTraits<KV>::EB;
  uint4 k[Frag<KV, D>::NLOAD * Frag<KV, D>::QCH];
  uint32_t vf[Frag<KV, D>::NT][QB];
  uint32_t vs[Frag<KV, D>::NLOAD][X / 4];
};

template <int KV, int D>
__device__ __forceinline__ void load_append_regs(const DecodeArgs& a, int s, int g, int lane,
                                                 AppendRegs<KV, D>& r) {
  using F = Frag<KV, D>;
  constexpr int QB = KvTraits<KV>::QB;
  constexpr int X = 16 / KvTraits<KV>::EB;
  const int row = lane >> 4, col = lane & 15;
  const uint8_t* kn = static_cast<const uint8_t*>(a.k_new) + (int64_t(s) * a.Hkv + g) * D * QB;
  const uint8_t* vn = static_cast<const uint8_t*>(a.v_new) + (int64_t(s) * a.Hkv + g) * D * QB;
#pragma unroll
  for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
    for (int c = 0; c < F::QCH; ++c)
      r.k[i * F::QCH + c] = *reinterpret_cast<const uint4*>(kn + (X * (4 * i + row)) * QB + 16 * c);
#pragma unroll
  for (int n = 0; n < F::NT; ++n) {
    const uint8_t* src = vn + (16 * n + 4 * row) * QB;
    if constexpr (QB == 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(src);
      r.vf[n][0] = w.x; r.vf[n][1] = w.y; r.vf[n][2] = w.z; r.vf[n][3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(src);
      r.vf[n][0] = w.x; r.vf[n][1] = w.y;
    }
  }
#pragma unroll
  for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
    for (int e = 0; e < X / 4; ++e) {
      const int d = i * 4 * X + 16 * e + col;
      r.vs[i][e] = QB == 4 ? reinterpret_cast<const uint32_t*>(vn)[d] : reinterpret_cast<const uint16_t*>(vn)[d];
    }
}

// Folds the appended token into the running softmax of head lane % 16: its logit from this
// lane's q fragments and the key as the cache holds it (summed over the four lane rows),
// then m, the sum and the accumulators as for a cached token; the probability is rounded
// to bf16 for the bf16 / fp8 accumulators, as the matrix path rounds it.  `zero` stands for
// an appended slot in a block outside the pool, which reads as zeros.
template <int KV, int D>
__device__ __forceinline__ void fold_append_token(const DecodeArgs& a, const AppendRegs<KV, D>& r,
                                                  const uint4* qf, int lane, bool zero, float& m_run,
                                                  float& l_run, f32x4* acc) {
  using F = Frag<KV, D>;
  constexpr int QB = KvTraits<KV>::QB;
  constexpr int X = 16 / KvTraits<KV>::EB;
  const int row = lane >> 4;
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
    for (int e = 0; e < X; ++e) {
      const uint32_t kx = input_element<QB>(r.k + i * F::QCH, e);
      const uint32_t qx = input_element<QB>(qf + i * F::QCH, e);
      const float qv = QB == 4 ? __uint_as_float(qx) : pkv::bf16_bits_to_f32(qx);
      dot += qv * cache_value<KV>(cache_bits<KV>(kx, a.k_inv));
    }
  dot += __shfl_xor(dot, 16);
  dot += __shfl_xor(dot, 32);
  const float sc = zero ? 0.f : dot * a.qk_scale_log2;
  const float m_new = fmaxf(m_run, sc);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  const float pr = __builtin_amdgcn_exp2f(sc - m_new);
  l_run = l_run * alpha + (row == 0 ? pr : 0.f);
  const float pm = zero ? 0.f : (KV == PKV_F32 ? pr : __uint_as_float(bf16_rne(pr) << 16));
#pragma unroll
  for (int n = 0; n < F::NT; ++n)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = QB == 4 ? r.vf[n][j] : (r.vf[n][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      acc[n][j] = acc[n][j] * alpha + pm * cache_value<KV>(cache_bits<KV>(x, a.v_inv));
    }
  m_run = m_new;
}

// The appended token's bytes this lane stores, in the cache's format: the K chunk of load
// i (lanes with lane % 16 == t) and its element of the V chunk of load i (lanes with
// lane / 16 == t / 4, at position e*4 + t%4).
template <int KV, int D>
struct AppendStore {
  uint4 k[Frag<KV, D>::NLOAD];
  uint32_t v[Frag<KV, D>::NLOAD][16 / KvTraits<KV>::EB / 4];
  int64_t sub = -1;  // byte offset of the sub-tile's K / V region in the pools; -1 = none
  int t = 0;         // token within the sub-tile
};

template <int KV, int D>
__device__ __forceinline__ void make_append_store(const DecodeArgs& a, const AppendRegs<KV, D>& r,
                                                  int64_t sub, int t, AppendStore<KV, D>& st) {
  using F = Frag<KV, D>;
  constexpr int EB = KvTraits<KV>::EB;
  constexpr int QB = KvTraits<KV>::QB;
  constexpr int X = 16 / EB;
#pragma unroll
  for (int i = 0; i < F::NLOAD; ++i) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < X; ++e)
      w[(e * EB) >> 2] |= cache_bits<KV>(input_element<QB>(r.k + i * F::QCH, e), a.k_inv) << (8 * ((e * EB) & 3));
    st.k[i] = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
    for (int e = 0; e < X / 4; ++e) st.v[i][e] = cache_bits<KV>(r.vs[i][e], a.v_inv);
  }
  st.sub = sub;
  st.t = t;
}

template <int KV, int D>
__device__ __forceinline__ void issue_append_store(const DecodeArgs& a, const AppendStore<KV, D>& st,
                                                   int lane) {
  using F = Frag<KV, D>;
  constexpr int EB = KvTraits<KV>::EB;
  constexpr int X = 16 / EB;
  uint8_t* ksub = a.k_cache_w + st.sub;
  uint8_t* vsub = a.v_cache_w + st.sub;
  if ((lane & 15) == st.t) {
#pragma unroll
    for (int i = 0; i < F::NLOAD; ++i) *reinterpret_cast<uint4*>(ksub + (64 * i + lane) * 16) = st.k[i];
  }
  if ((lane >> 4) == (st.t >> 2)) {
#pragma unroll
    for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
      for (int e = 0; e < X / 4; ++e) {
        uint8_t* dst = vsub + (64 * i + lane) * 16 + (e * 4 + (st.t & 3)) * EB;
        if constexpr (EB == 4)
          *reinterpret_cast<uint32_t*>(dst) = st.v[i][e];
        else if constexpr (EB == 2)
          *reinterpret_cast<uint16_t*>(dst) = uint16_t(st.v[i][e]);
        else
          *dst = uint8_t(st.v[i][e]);
      }
  }
}

// Partial (accumulator, max, sum) of one column into row r of a piece array (D floats per row
// of acc_base, two per row of ml_base); lane (column, row) holds dims 16*n + 4*row .. +3 of
// each 16-dim tile n.
template <int D>
__device__ __forceinline__ void store_row(float* acc_base, float* ml_base, int64_t r, int row, const f32x4* acc,
                                          float2 ml) {
  float* wacc = acc_base + r * D;
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    *reinterpret_cast<float4*>(wacc + 16 * n + 4 * row) = make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
  if (row == 0) *reinterpret_cast<float2*>(ml_base + r * 2) = ml;
}

// Partial of head h of piece `piece`.
template <int D>
__device__ __forceinline__ void store_partial(const DecodeArgs& a, int64_t piece, int h, int row, const f32x4* acc,
                                              float2 ml) {
  store_row<D>(a.ws_acc, a.ws_ml, piece * a.G + h, row, acc, ml);
}

// One share of the (sequence, head group, block) work list: positions [c_begin, c_end),
// walked by wave `sub` of the share's group of `coop` waves on kv heads coop * hg + sub, so
// that together they read the adjacent head regions of each block.  The share's pieces are
// numbered (share * coop + sub) * 2 + slot.
//  CONTIG: the sequence's blocks are consecutive pool blocks from seq_first_block[s] on, so a
//    block's address is computed instead of looked up (no table loads).
//  GROUPED: the list holds each sequence's blocks after the leading ones the group pass reads
//    for it; a unit finished inside the share goes to its (sequence, kv head) slot instead of
//    `out` when the group pass also holds part of it.
// hold / hold_ml: this wave's LDS rows for the partial of the share's first segment.
template <int KV, int D, int BS, int NSUB, bool APPEND, bool MIX, bool CONTIG, bool GROUPED>
__device__ __forceinline__ void split_walk(const DecodeArgs& a, int lane, int share, int sub, int c_begin,
                                           int c_end, f32x4 (*hold)[64], float2* hold_ml,
                                           const int* lds_off = nullptr, const int* lds_len = nullptr,
                                           int s_start = 0, int off_start = 0) {
  static_assert(!(CONTIG && APPEND), "the contiguous placement has no decode step with append");
  static_assert(!(GROUPED && (MIX || CONTIG)), "prefix groups read shared blocks once, through tables");
  using F = Frag<KV, D>;
  using T = KvTraits<KV>;
  constexpr int X = 16 / T::EB;                  // cached elements per 16-byte chunk
  constexpr int SUB_BYTES = 16 * D * T::EB;       // one 16-token sub-tile
  constexpr int NSB = BS / 16;                    // sub-tiles per block
  constexpr int64_t REGION = int64_t(BS) * D * T::EB;

  bool holding = false;
  // lds_off / lds_len (when the workgroup has scanned the list): exclusive prefix sums of the
  // per-unit spans of the list and the sequences' clamped lengths, in LDS, and the share's
  // first sequence and its offset, found there.  A unit's blocks then follow from its span.
  int s, seq_off;
  if (lds_off) {
    s = s_start;
    seq_off = off_start;
  } else {
    locate<GROUPED>(a, BS, lane, c_begin, s, seq_off);
  }
  if (s >= a.B) return;
  int L = lds_len ? lds_len[s] : seq_len(a, s, BS);
  int nbt = (L + BS - 1) / BS;                     // blocks of the sequence
  int skip, nb;                                    // leading blocks the group pass reads; blocks
  if (lds_off) {                                   // of each of its units in this list
    nb = (lds_off[s + 1] - lds_off[s] - kUnitW) / kBlockW;
    skip = nbt - nb;
  } else {
    skip = GROUPED ? group_skip(a, s, BS) : 0;
    nb = nbt - skip;
  }
  int span = unit_span(nb, kBlockW);
  int hg = (c_begin - seq_off) / span;
  int g = hg * a.coop + sub;
  int unit_off = seq_off + hg * span;
  int pos = c_begin;
  bool done = false;
  // Next unit: next kv head of this sequence, else the next sequence with blocks in the list.
  auto next_unit = [&]() {
    unit_off += span;
    if (++hg == head_groups(a)) {
      hg = 0;
      if (lds_off) {
        do {
          done = ++s >= a.B;
        } while (!done && lds_off[s + 1] == lds_off[s]);
      } else {
        do {
          done = ++s >= a.B;
        } while (!done && unit_blocks<GROUPED>(a, s, BS) == 0);
      }
      if (done) return false;
      L = lds_len ? lds_len[s] : seq_len(a, s, BS);
      nbt = (L + BS - 1) / BS;
      if (lds_off) {
        nb = (lds_off[s + 1] - lds_off[s] - kUnitW) / kBlockW;
        skip = nbt - nb;
      } else {
        skip = GROUPED ? group_skip(a, s, BS) : 0;
        nb = nbt - skip;
      }
      span = unit_span(nb, kBlockW);
    }
    g = hg * a.coop + sub;
    return true;
  };

  const int h = lane & 15;       // head (within the group) of this lane's QK/PV column
  const int row = lane >> 4;     // token group 4*row.. of this lane's QK/PV rows
  const bool head_ok = h < a.G;

  // With APPEND, token L-1 of every sequence is the appended one.  The block walk masks its
  // slot (Lc = L - 1 cached tokens are read); the segment that ends the unit loads the
  // token's k_new / v_new values when it starts, folds the token in after the walk and keeps
  // its pool stores in registers until the wave has issued its last load: a wave's loads and
  // stores complete in issue order, so a store ahead of the remaining loads would delay them.
  AppendStore<KV, D> held;
  while (pos < c_end) {
    const int Lc = APPEND ? L - 1 : L;
    const int unit_end = unit_off + span;
    const int seg_end = std::min(c_end, unit_end);
    int r0, r1;                                       // the unit's blocks this share holds
    unit_blocks_in(unit_off, nb, kBlockW, c_begin, c_end, r0, r1);
    if (r1 <= r0) {                                   // none: the share ends or starts in this
      pos = seg_end;                                  // unit's weight without a block start
      if (pos >= c_end || !next_unit()) break;
      continue;
    }
    const bool full = r0 == 0 && r1 == nb;
    const int j0 = skip + r0, j1 = skip + r1;         // blocks [j0, j1) of the sequence
    const int k0 = j0 * NSB;
    const int k1 = (std::min(j1 * BS, Lc) + 15) / 16;                   // sub-tiles [k0, k1)
    // Sub-tiles below ks lie in blocks shared with other sequences: cached loads.
    const int ks = MIX ? std::min(__builtin_amdgcn_readfirstlane(a.shared_prefix[s]), nbt) * NSB : 0;

    // q fragments of (s, g): lane (h, row) holds q[s, g*G+h, X*(4i+row) .. +X].
    uint4 qf[F::NLOAD * F::QCH];
    {
      const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                            (int64_t(s) * a.Hkv * a.G + int64_t(g) * a.G + h) * D * T::QB;
#pragma unroll
      for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
        for (int c = 0; c < F::QCH; ++c)
          qf[i * F::QCH + c] = head_ok ? *reinterpret_cast<const uint4*>(
                                             qrow + (int64_t(X) * (4 * i + row)) * T::QB + 16 * c)
                                       : make_uint4(0u, 0u, 0u, 0u);
    }

    // The first window of block-table entries is requested together with q, so that both
    // arrive in one round trip.
    const int32_t* trow = CONTIG ? nullptr : a.block_tables + int64_t(s) * a.max_blocks;
    int tbase = k0 / NSB;
    int tbl = -1;
    int first = 0;
    if constexpr (CONTIG) first = __builtin_amdgcn_readfirstlane(a.seq_first_block[s]);
    else tbl = tbase + lane < nbt ? trow[tbase + lane] : -1;
    const bool ends_unit = APPEND && r1 == nb;
    AppendRegs<KV, D> app;
    if constexpr (APPEND) {
      if (ends_unit) load_append_regs<KV, D>(a, s, g, lane, app);
    }
    f32x4 acc[F::NT];
#pragma unroll
    for (int n = 0; n < F::NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const uint8_t* kbase = a.k_cache + int64_t(g) * REGION;
    const uint8_t* vbase = a.v_cache + int64_t(g) * REGION;
    const int64_t block_stride = int64_t(a.Hkv) * REGION;

    for (int k = k0; k < k1; k += NSUB) {
      const int cnt = std::min(NSUB, k1 - k);
      const int jlast = (k + cnt - 1) / NSB;
      if (!CONTIG && (k / NSB < tbase || jlast >= tbase + 64)) {
        tbase = k / NSB;
        const int jj = tbase + lane;
        tbl = jj < nbt ? trow[jj] : -1;
      }
      // Issue every K load of the chunk, then every V load, with no branches between
      // them, so QK can start while V is still in flight.  Sub-tiles past the chunk's
      // end re-read its first sub-tile (a cache hit, never used).  A table entry outside
      // [0, num_blocks) reads block 0 instead and its keys and values are replaced by
      // zeros where they are used.
      uint4 kf[NSUB][F::NLOAD], vf[NSUB][F::NLOAD];
      int64_t off[NSUB];
      bool bad[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int ku = u < cnt ? k + u : k;
        const int64_t phys = CONTIG ? int64_t(first) + ku / NSB
                                    : int64_t(__builtin_amdgcn_readlane(tbl, (ku / NSB - tbase) & 63));
        bad[u] = uint64_t(phys) >= uint64_t(a.num_blocks);
        off[u] = (bad[u] ? 0 : phys * block_stride) + (ku % NSB) * SUB_BYTES + lane * 16;
      }
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i)
          kf[u][i] = load_kv(kbase + off[u] + i * 1024, MIX && k + u < ks);
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i)
          vf[u][i] = load_kv(vbase + off[u] + i * 1024, MIX && k + u < ks);
      // Everything below is branch-free on the loaded data: a branch around QK or PV
      // would let the compiler sink the chunk loads into it and wait on them one by one.
      // Sub-tiles past the chunk's end and out-of-range blocks are masked instead: their
      // K chunks are zeroed (a block outside the pool reads as zeros), their scores are
      // -inf past the context or the chunk, and their V elements are zeroed.
      float sc[NSUB][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int tok0 = (k + u) * 16 + 4 * row;
        const uint32_t km = bad[u] ? 0u : 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i) {
          kf[u][i].x &= km; kf[u][i].y &= km; kf[u][i].z &= km; kf[u][i].w &= km;
        }
        const f32x4 c = qk_subtile<KV, D>(kf[u], qf);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sc[u][j] = (u < cnt && tok0 + j < Lc) ? c[j] * a.qk_scale_log2 : -INFINITY;
          cmax = fmaxf(cmax, sc[u][j]);
        }
      }
      cmax = wave_max_rows(cmax);
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < F::NT; ++n) acc[n] *= alpha;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int tok0 = (k + u) * 16 + 4 * row;
        float p[4];
        uint32_t vm = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = __builtin_amdgcn_exp2f(sc[u][j] - m_new);   // 0 where masked
          l_run += p[j];
          vm |= (u < cnt && tok0 + j < Lc && !bad[u] ? 1u : 0u) << j;
        }
        mask_v<KV, D>(vf[u], vm);
        pv_subtile<KV, D>(acc, vf[u], p);
      }
    }

    if constexpr (APPEND) {
      if (ends_unit) {
        const int knew = (L - 1) / 16;
        const int jb = knew / NSB;   // usually inside the walk's last table window
        const int phys = jb >= tbase && jb < tbase + 64 ? __builtin_amdgcn_readlane(tbl, jb - tbase) : trow[jb];
        const bool zero = unsigned(phys) >= unsigned(a.num_blocks);
        fold_append_token<KV, D>(a, app, qf, lane, zero, m_run, l_run, acc);
        if (held.sub >= 0) issue_append_store<KV, D>(a, held, lane);   // a second unit end
        held.sub = -1;
        if (!zero)
          make_append_store<KV, D>(a, app, int64_t(phys) * block_stride + int64_t(g) * REGION +
                                               (knew % NSB) * SUB_BYTES,
                                   (L - 1) & 15, held);
      }
    }
    const float l_tot = wave_sum_rows(l_run);
    if (GROUPED && full && skip > 0) {
      // The group pass holds the rest of this (sequence, kv head): the merge combines them.
      if (head_ok) store_row<D>(a.ws_macc, a.ws_mml, (int64_t(s) * a.Hkv + g) * a.G + h, row, acc,
                                make_float2(m_run, l_tot));
    } else if (full) {
      if (head_ok) {
        const float inv = a.v_scale / l_tot;
        const int64_t orow = (int64_t(s) * a.Hkv * a.G + int64_t(g) * a.G + h) * D;
#pragma unroll
        for (int n = 0; n < F::NT; ++n) {
          const int d = 16 * n + 4 * row;
          if constexpr (KV == PKV_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d) =
                make_float4(acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv, acc[n][3] * inv);
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d) =
                make_uint2(pack_bf16x2(acc[n][0] * inv, acc[n][1] * inv),
                           pack_bf16x2(acc[n][2] * inv, acc[n][3] * inv));
          }
        }
      }
    } else {
      // The share's first segment (it begins within this unit's weight) waits in LDS; any
      // other unfinished segment is the share's last.
      const int slot = c_begin >= unit_off ? 0 : 1;
      if (slot == 0) {
#pragma unroll
        for (int n = 0; n < F::NT; ++n) hold[n][lane] = acc[n];
        hold_ml[lane] = make_float2(m_run, l_tot);
        holding = true;
      } else if (head_ok) {
        store_partial<D>(a, (int64_t(share) * a.coop + sub) * 2 + 1, h, row, acc, make_float2(m_run, l_tot));
      }
    }

    pos = seg_end;
    if (pos >= c_end || !next_unit()) break;
  }

  if (holding && head_ok) {
    f32x4 acc[F::NT];
#pragma unroll
    for (int n = 0; n < F::NT; ++n) acc[n] = hold[n][lane];
    store_partial<D>(a, (int64_t(share) * a.coop + sub) * 2, h, row, acc, hold_ml[lane]);
  }
  if constexpr (APPEND) {
    if (held.sub >= 0) issue_append_store<KV, D>(a, held, lane);
  }
}

// Logical wave of this lane's wave.  Workgroup b runs on XCD b % 8; each XCD takes a contiguous
// eighth of the work list (logical workgroup (b % 8) * (n / 8) + b / 8), so sequences next to
// each other, such as the members of a group that share prefix blocks, read those blocks
// through one XCD's L2 at about the same time.  Shares and pieces are numbered by the logical
// wave.
__device__ __forceinline__ int logical_wave(int wv) {
  const int nwg = int(gridDim.x), full = nwg - nwg % kXcds;
  const int b = int(blockIdx.x);
  const int lwg = b < full ? (b % kXcds) * (full / kXcds) + b / kXcds : b;
  return lwg * kWavesPerWG + wv;
}

// Writes every sequence's offset in a work list ([B], then the total at [B]) for the merge.
// GROUP: the group work list (chunk first sequences).
template <bool GROUPED, bool GROUP>
__device__ __forceinline__ void write_offsets(const DecodeArgs& a, int bs, int lane, int* dst) {
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int sq = b0 + lane;
    const int w = sq < a.B ? (GROUP ? unit_span(chunk_blocks(a, sq, bs), kGroupBlockW)
                                    : unit_span(unit_blocks<GROUPED>(a, sq, bs), kBlockW)) * head_groups(a)
                           : 0;
    const int incl = wave_incl_scan(w, lane);
    if (sq < a.B) dst[sq] = base + incl - w;
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) dst[a.B] = base;
}

template <int KV, int D, int BS, int NSUB, bool APPEND, bool MIX, bool CONTIG = false>
__global__ __launch_bounds__(kWavesPerWG * 64, 2) void paged_attention_split_kernel(DecodeArgs a) {
  using F = Frag<KV, D>;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = logical_wave(wv);
  // The partial of a share's first segment waits in LDS until the share's loads are done: a
  // wave's loads and stores complete in issue order, so a store in the middle of the share
  // would hold up every load behind it.  Each lane reads back only what it wrote.
  __shared__ f32x4 s_hold[kWavesPerWG][F::NT][64];
  __shared__ float2 s_hold_ml[kWavesPerWG][64];
  // The work list, scanned by the workgroup when the batch fits (as in the prefix-group
  // pass): exclusive prefix sums of the per-unit spans ([B] on: the total) and the clamped
  // lengths.
  __shared__ int s_off[kScanSeqs + 1];
  __shared__ int s_len[kScanSeqs];
  __shared__ int s_wsum[kWavesPerWG];
  const int hg = head_groups(a);
  const bool lds_lists = a.B <= kScanSeqs;
  int W;
  if (lds_lists) {
    const int tid = threadIdx.x;
    int len[kScanPerThread], sp[kScanPerThread], sum = 0;
#pragma unroll
    for (int r = 0; r < kScanPerThread; ++r) {
      const int sq = tid * kScanPerThread + r;
      const int L = seq_len(a, std::min(sq, a.B - 1), BS);
      len[r] = sq < a.B ? L : 0;
      sp[r] = unit_span((len[r] + BS - 1) / BS, kBlockW);
      sum += sp[r];
    }
    const int incl = wave_incl_scan(sum, lane);
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int base = incl - sum, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) {
      base += w < wv ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
#pragma unroll
    for (int r = 0; r < kScanPerThread; ++r) {
      const int sq = tid * kScanPerThread + r;
      s_off[sq] = base;
      s_len[sq] = len[r];
      base += sp[r];
    }
    if (tid == 0) s_off[kScanSeqs] = total;
    __syncthreads();
    W = total * hg;
  } else {
    W = total_work(a, BS, lane);
  }
  if (wave == 0) {
    if (lds_lists) {
      for (int sq = lane; sq <= a.B; sq += 64) a.ws_seq[sq] = s_off[sq] * hg;
    } else {
      write_offsets<false, false>(a, BS, lane, a.ws_seq);
    }
    if (lane == 0) {
      a.ws_seq[a.B + 1] = a.splits;
      a.ws_seq[a.B + 2] = a.coop;
      a.ws_seq[a.B + 3] = a.B;
    }
  }
  if (W == 0) return;
  const int share = wave / a.coop;
  const int sub = wave % a.coop;
  const int nshare = list_shares(a.splits / a.coop, W, kBlockW);
  if (share >= nshare) return;
  const int c_begin = __builtin_amdgcn_readfirstlane(int(share_begin(share, W, nshare)));
  const int c_end = __builtin_amdgcn_readfirstlane(int(share_begin(share + 1, W, nshare)));
  int s0 = 0, off0 = 0;
  if (lds_lists) {
    s0 = __builtin_amdgcn_readfirstlane(lds_search(s_off, a.B, hg, c_begin, lane));
    off0 = s_off[s0] * hg;
  }
  split_walk<KV, D, BS, NSUB, APPEND, MIX, CONTIG, false>(a, lane, share, sub, c_begin, c_end, s_hold[wv],
                                                          s_hold_ml[wv], lds_lists ? s_off : nullptr,
                                                          lds_lists ? s_len : nullptr, s0, off0);
}

// One share of the group work list (chunk first sequence f, head group, block j < P_f):
// positions [c_begin, c_end) of W.  A chunk's shared blocks come from its source sequence's
// table and are read once for all its members: the 32 columns are (member m, query head h) =
// (c / G, c % G) for the members f + m of the chunk, in two 16-column tiles, each column
// masked to the tokens of its member's own shared blocks.  Every segment leaves a partial per
// column: a unit finished inside the share in its (f, kv head) slot, the share's first and
// last segments as pieces (share * coop + sub) * 2 + slot.
template <int KV, int D, int BS>
__device__ __forceinline__ void group_walk(const DecodeArgs& a, int lane, int share, int sub, int c_begin, int c_end,
                                           f32x4 (*hold)[64], float2 (*hold_ml)[64], const int* lds_off = nullptr,
                                           const int* lds_glim = nullptr, int f_start = 0, int off_start = 0) {
  using F = Frag<KV, D>;
  using T = KvTraits<KV>;
  constexpr int X = 16 / T::EB;
  constexpr int SUB_BYTES = 16 * D * T::EB;
  constexpr int NSB = BS / 16;
  constexpr int64_t REGION = int64_t(BS) * D * T::EB;
  constexpr int CT = kGroupCols / 16;
  const int M = kGroupCols / a.G;
  const int row = lane >> 4;
  bool holding = false;

  // lds_off: as in split_walk, over the group list's per-unit spans; lds_glim: every
  // sequence's chunk and group blocks (kNoChunk and the group blocks' entry layout above).
  int f, chunk_off;
  if (lds_off) {
    f = f_start;
    chunk_off = off_start;
  } else {
    locate<false, true>(a, BS, lane, c_begin, f, chunk_off);
  }
  if (f >= a.B) return;
  int P = lds_off ? (lds_off[f + 1] - lds_off[f] - kUnitW) / kGroupBlockW : chunk_blocks(a, f, BS);
  int span = unit_span(P, kGroupBlockW);
  int hg = (c_begin - chunk_off) / span;
  int g = hg * a.coop + sub;
  int unit_off = chunk_off + hg * span;
  int pos = c_begin;
  const int64_t block_stride = int64_t(a.Hkv) * REGION;
  // Next unit: next kv-head group of this chunk, else the next chunk with blocks to read.
  auto next_unit = [&]() {
    unit_off += span;
    if (++hg == head_groups(a)) {
      hg = 0;
      if (lds_off) {
        do {
          ++f;
        } while (f < a.B && lds_off[f + 1] == lds_off[f]);
        if (f >= a.B) return false;
        P = (lds_off[f + 1] - lds_off[f] - kUnitW) / kGroupBlockW;
      } else {
        do {
          ++f;
        } while (f < a.B && chunk_blocks(a, f, BS) == 0);
        if (f >= a.B) return false;
        P = chunk_blocks(a, f, BS);
      }
      span = unit_span(P, kGroupBlockW);
    }
    g = hg * a.coop + sub;
    return true;
  };

  while (pos < c_end) {
    const int seg_end = std::min(c_end, unit_off + span);
    int r0, r1;                                       // the unit's blocks this share holds
    unit_blocks_in(unit_off, P, kGroupBlockW, c_begin, c_end, r0, r1);
    if (r1 <= r0) {
      pos = seg_end;
      if (pos >= c_end || !next_unit()) break;
      continue;
    }
    const bool full = r0 == 0 && r1 == P;
    const int k0 = r0 * NSB, k1 = r1 * NSB;           // whole blocks
    // Columns: this lane's member and head in each tile, its token limit and q fragments.
    int lim[CT];
    uint4 qf[CT][F::NLOAD * F::QCH];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + (lane & 15);
      const int m = c / a.G, hh = c % a.G, sq = f + m;
      if (lds_glim) {
        const int gl = m < M && sq < a.B ? lds_glim[sq] : kNoChunk;
        lim[ct] = (gl & kNoChunk) == f ? (gl >> 10) * BS : 0;
      } else {
        const bool member = m < M && sq < a.B && a.chunk_first[sq] == f;
        lim[ct] = member ? group_skip(a, sq, BS) * BS : 0;
      }
      const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                            ((int64_t(sq) * a.Hkv + g) * a.G + hh) * D * T::QB;
#pragma unroll
      for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
        for (int cc = 0; cc < F::QCH; ++cc)
          qf[ct][i * F::QCH + cc] =
              lim[ct] > 0 ? *reinterpret_cast<const uint4*>(qrow + (int64_t(X) * (4 * i + row)) * T::QB + 16 * cc)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
    const int32_t* trow = a.block_tables + int64_t(__builtin_amdgcn_readfirstlane(a.chunk_src[f])) * a.max_blocks;
    int tbase = k0 / NSB;
    int tbl = tbase + lane < P ? trow[tbase + lane] : -1;
    f32x4 acc[CT][F::NT];
    float m_run[CT], l_run[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int n = 0; n < F::NT; ++n) acc[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[ct] = -INFINITY;
      l_run[ct] = 0.f;
    }
    const uint8_t* kbase = a.k_cache + int64_t(g) * REGION;
    const uint8_t* vbase = a.v_cache + int64_t(g) * REGION;

    for (int k = k0; k < k1; ++k) {
      if (k / NSB >= tbase + 64) {
        tbase = k / NSB;
        tbl = tbase + lane < P ? trow[tbase + lane] : -1;
      }
      // K and V of the sub-tile, loaded together with no branch before their use; a table
      // entry outside [0, num_blocks) reads block 0, whose keys and values are zeroed.
      const int phys = __builtin_amdgcn_readlane(tbl, k / NSB - tbase);
      const bool bad = unsigned(phys) >= unsigned(a.num_blocks);
      const int64_t off = (bad ? 0 : int64_t(phys) * block_stride) + (k % NSB) * SUB_BYTES + lane * 16;
      uint4 kf[F::NLOAD], vf[F::NLOAD];
#pragma unroll
      for (int i = 0; i < F::NLOAD; ++i) kf[i] = load_stream(kbase + off + i * 1024);
#pragma unroll
      for (int i = 0; i < F::NLOAD; ++i) vf[i] = load_stream(vbase + off + i * 1024);
      const uint32_t km = bad ? 0u : 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < F::NLOAD; ++i) {
        kf[i].x &= km; kf[i].y &= km; kf[i].z &= km; kf[i].w &= km;
      }
      const int t0 = k * 16 + 4 * row;
      float p[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const f32x4 c = qk_subtile<KV, D>(kf, qf[ct]);
        float sc[4];
        float cmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sc[j] = t0 + j < lim[ct] ? c[j] * a.qk_scale_log2 : -INFINITY;
          cmax = fmaxf(cmax, sc[j]);
        }
        cmax = wave_max_rows(cmax);
        const float m_new = fmaxf(m_run[ct], cmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;   // a column with no token yet
        const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_use);
        m_run[ct] = m_new;
        l_run[ct] *= alpha;
#pragma unroll
        for (int n = 0; n < F::NT; ++n) acc[ct][n] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[ct][j] = __builtin_amdgcn_exp2f(sc[j] - m_use);        // 0 where masked
          l_run[ct] += p[ct][j];
        }
      }
      mask_v<KV, D>(vf, bad ? 0u : 0xFu);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) pv_subtile<KV, D>(acc[ct], vf, p[ct]);
    }

    const int slot = c_begin >= unit_off ? 0 : 1;   // first segment of the share, or its last
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float l_tot = wave_sum_rows(l_run[ct]);
      const int c = 16 * ct + (lane & 15);
      if (full) {
        store_row<D>(a.ws_fgacc, a.ws_fgml, (int64_t(f) * a.Hkv + g) * kGroupCols + c, row, acc[ct],
                     make_float2(m_run[ct], l_tot));
      } else if (slot == 0) {
#pragma unroll
        for (int n = 0; n < F::NT; ++n) hold[ct * F::NT + n][lane] = acc[ct][n];
        hold_ml[ct][lane] = make_float2(m_run[ct], l_tot);
      } else {
        store_row<D>(a.ws_gacc, a.ws_gml, ((int64_t(share) * a.coop + sub) * 2 + 1) * kGroupCols + c, row, acc[ct],
                     make_float2(m_run[ct], l_tot));
      }
    }
    if (slot == 0 && !full) holding = true;

    pos = seg_end;
    if (pos >= c_end || !next_unit()) break;
  }
  if (holding) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 acc[F::NT];
#pragma unroll
      for (int n = 0; n < F::NT; ++n) acc[n] = hold[ct * F::NT + n][lane];
      store_row<D>(a.ws_gacc, a.ws_gml, ((int64_t(share) * a.coop + sub) * 2) * kGroupCols + 16 * ct + (lane & 15), row,
                   acc, hold_ml[ct][lane]);
    }
  }
}

// Share counts of a grouped launch: S shares in all, nsg of them over the group work list
// (in proportion to its weighted positions, at least one when it has any) and the rest over
// the member work list; neither list gets a share shorter than one of its blocks' weight.
__device__ __forceinline__ void grouped_shares(const DecodeArgs& a, int Wm, int Wg, int& S, int& nsg) {
  const int max_g = Wg / kGroupBlockW, max_m = Wm / kBlockW;   // shares no shorter than a block
  S = std::min(a.splits / a.coop, max_g + max_m);
  nsg = 0;
  if (Wg > 0) {
    nsg = Wm == 0 ? S : int((int64_t(S) * Wg + (Wm + Wg) / 2) / (Wm + Wg));
    nsg = std::min(std::max(nsg, 1), max_g);
    nsg = std::min(nsg, S - (Wm > 0 ? 1 : 0));
    nsg = std::max(nsg, S - max_m);
  }
}

// The split pass with prefix groups: each share is a group share or a member share, spread
// evenly over the launch (share w is a group share when floor((w+1) nsg / S) exceeds
// floor(w nsg / S)), so that both kinds run on every XCD at once.  Header: member offsets
// [B+1] (total at [B]), the split count, head-group width and B at [B+1..B+3], group offsets
// [B+1] from [B+4] (total at [2B+4]), nsg at [2B+5].
// Start-up: with at most kScanSeqs sequences, the workgroup's threads take the sequences
// between them, each with its lookups in flight together, and scan both lists into LDS; a
// wave then finds its share's first unit there and reads later units' block counts there,
// instead of walking the sequences' entries 64 at a time through dependent loads.
template <int KV, int D, int BS, int NSUB, bool APPEND>
__global__ __launch_bounds__(kWavesPerWG * 64, 2) void paged_attention_grouped_kernel(DecodeArgs a) {
  using F = Frag<KV, D>;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = logical_wave(wv);
  __shared__ f32x4 s_hold[kWavesPerWG][(kGroupCols / 16) * F::NT][64];
  __shared__ float2 s_hold_ml[kWavesPerWG][kGroupCols / 16][64];
  // Both work lists, scanned by the workgroup when the batch fits: exclusive prefix sums of
  // the per-unit spans, [s] for sequence s and the total from [B] on.
  __shared__ int s_moff[kScanSeqs + 1];
  __shared__ int s_goff[kScanSeqs + 1];
  __shared__ int s_len[kScanSeqs];
  __shared__ int s_glim[kScanSeqs];
  __shared__ int s_wsum[2][kWavesPerWG];
  const int hg = head_groups(a);
  const bool lds_lists = a.B <= kScanSeqs;
  // (Neither these entries nor the LDS lengths for f32 caches, whose appending kernel has no
  // registers to spare for them.)
  const bool lds_glim = KV != PKV_F32 && lds_lists && a.max_blocks < kGlimMaxBlocks;
  int Wm, Wg;
  if (lds_lists) {
    const int tid = threadIdx.x;
    SeqSpans sp[kScanPerThread];
    int ms[kScanPerThread], gs[kScanPerThread];
    int msum = 0, gsum = 0;
#pragma unroll
    for (int r = 0; r < kScanPerThread; ++r) {
      const int sq = tid * kScanPerThread + r;
      sp[r] = seq_spans(a, std::min(sq, a.B - 1), BS);
      ms[r] = sq < a.B ? sp[r].mspan : 0;
      gs[r] = sq < a.B ? sp[r].gspan : 0;
      msum += ms[r];
      gsum += gs[r];
    }
    const int mi = wave_incl_scan(msum, lane), gi = wave_incl_scan(gsum, lane);
    if (lane == 63) {
      s_wsum[0][wv] = mi;
      s_wsum[1][wv] = gi;
    }
    __syncthreads();
    int mb = mi - msum, gb = gi - gsum, mt = 0, gt = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) {
      mb += w < wv ? s_wsum[0][w] : 0;
      gb += w < wv ? s_wsum[1][w] : 0;
      mt += s_wsum[0][w];
      gt += s_wsum[1][w];
    }
#pragma unroll
    for (int r = 0; r < kScanPerThread; ++r) {
      const int sq = tid * kScanPerThread + r;
      s_moff[sq] = mb;
      s_goff[sq] = gb;
      s_len[sq] = sp[r].L;
      s_glim[sq] = int((unsigned(sp[r].skip) << 10) | (unsigned(sp[r].cf) < unsigned(a.B) ? sp[r].cf : kNoChunk));
      mb += ms[r];
      gb += gs[r];
    }
    if (tid == 0) {
      s_moff[kScanSeqs] = mt;
      s_goff[kScanSeqs] = gt;
    }
    __syncthreads();
    Wm = mt * hg;
    Wg = gt * hg;
    if (blockIdx.x == 0) {
#pragma unroll
      for (int r = 0; r < kScanPerThread; ++r) {
        const int sq = tid * kScanPerThread + r;
        if (sq < a.B) {
          const bool grp = sp[r].skip > 0;
          int* rec = a.ws_rec + 8 * sq;
          *reinterpret_cast<int4*>(rec) = make_int4(s_moff[sq] * hg, grp ? s_goff[sp[r].f] * hg : 0, grp ? sp[r].P : 0,
                                                    sp[r].skip);
          *reinterpret_cast<int4*>(rec + 4) =
              make_int4(ms[r] > 0 ? (ms[r] - kUnitW) / kBlockW : 0, grp ? sp[r].f : 0, 0, 0);
        }
      }
    }
  } else {
    Wm = total_work<true>(a, BS, lane);
    Wg = group_work(a, BS, lane);
  }
  int S, nsg;
  grouped_shares(a, Wm, Wg, S, nsg);
  if (wave == 0) {
    if (lds_lists) {
      for (int sq = lane; sq <= a.B; sq += 64) {
        a.ws_seq[sq] = s_moff[sq] * hg;
        a.ws_seq[a.B + 4 + sq] = s_goff[sq] * hg;
      }
    } else {
      write_offsets<true, false>(a, BS, lane, a.ws_seq);
      write_offsets<false, true>(a, BS, lane, a.ws_seq + a.B + 4);
    }
    if (lane == 0) {
      a.ws_seq[a.B + 1] = a.splits;
      a.ws_seq[a.B + 2] = a.coop;
      a.ws_seq[a.B + 3] = a.B;
      a.ws_seq[2 * a.B + 5] = nsg;
    }
  }
  const int share = wave / a.coop;
  const int sub = wave % a.coop;
  if (share >= S) return;
  // Group share gi of nsg over Wg, or member share mi of S - nsg over Wm.  The share's index
  // and bounds are wave-uniform: kept in scalar registers.
  const int gi = int(int64_t(share) * nsg / S);
  const bool is_group = int64_t(share + 1) * nsg / S > gi;
  const int idx = __builtin_amdgcn_readfirstlane(is_group ? gi : share - gi);
  const int n = is_group ? nsg : S - nsg, Wl = is_group ? Wg : Wm;
  const int c_begin = __builtin_amdgcn_readfirstlane(int(share_begin(idx, Wl, n)));
  const int c_end = __builtin_amdgcn_readfirstlane(int(share_begin(idx + 1, Wl, n)));
  const int* lds_off = lds_lists ? (is_group ? s_goff : s_moff) : nullptr;
  int s0 = 0, off0 = 0;
  if (lds_lists) {
    s0 = __builtin_amdgcn_readfirstlane(lds_search(lds_off, a.B, hg, c_begin, lane));
    off0 = lds_off[s0] * hg;
  }
  if (is_group) {
    group_walk<KV, D, BS>(a, lane, idx, sub, c_begin, c_end, s_hold[wv], s_hold_ml[wv], lds_off,
                          lds_glim ? s_glim : nullptr, s0, off0);
  } else {
    split_walk<KV, D, BS, NSUB, APPEND, false, false, true>(a, lane, idx, sub, c_begin, c_end, s_hold[wv],
                                                            s_hold_ml[wv][0], lds_off,
                                                            KV != PKV_F32 && lds_lists ? s_len : nullptr, s0, off0);
  }
}

// One wave per (four query heads, sequence): merges the partials of a (sequence, kv head)
// unit that spans several shares, or writes zeros for an empty sequence.  Lanes 16*i ..
// 16*i+15 take head 4*hq + i of the group, each with D/16 consecutive dims, so a partial
// costs a lane two 16-byte loads and its head's (max, sum).  The unit's place in the work
// list comes from the offsets the split pass left in the workspace.  Partials are folded
// eight at a time with the running-softmax rule (load a batch's (max, sum) and accumulators
// together, raise the running max, rescale, add), and the next batch's loads are issued
// before the current batch is folded, so a unit with many partials (long contexts) keeps
// two batches in flight.
constexpr int kMergeHeads = 4;   // query heads per merge wave

// MW waves per workgroup (1, or 4 when units span many shares, as long contexts do): each
// wave folds a contiguous MW-th of the unit's pieces, and the waves' states meet in LDS.
constexpr int kMergeWavesLong = 4;
constexpr int kLongMergePieces = 16;   // shares per (sequence, kv-head group), at least, for MW = 4

template <int KV, int D, int BS, int MW>
__global__ __launch_bounds__(64 * MW) void paged_attention_merge_kernel(DecodeArgs a) {
  constexpr int EPL = D / 16;   // output dims per lane
  constexpr int BATCH = 8;      // partials per batch
  const int lane = threadIdx.x & 63;
  const int wv = MW == 1 ? 0 : __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  __shared__ float s_num[MW > 1 ? MW : 1][MW > 1 ? EPL : 1][64];
  __shared__ float2 s_md[MW > 1 ? MW : 1][64];
  const int hq_per_g = (a.G + kMergeHeads - 1) / kMergeHeads;
  const int g = blockIdx.x / hq_per_g, s = blockIdx.y;
  const int h_raw = (blockIdx.x % hq_per_g) * kMergeHeads + (lane >> 4);
  const bool head_ok = h_raw < a.G;
  const int h = head_ok ? h_raw : a.G - 1;   // idle lanes read a valid row and write nothing
  const int d0 = (lane & 15) * EPL;
  const int64_t orow = ((int64_t(s) * a.Hkv + g) * a.G + h) * D + d0;
  // The split pass's record: share count, head-group width, and where the partials lie.
  const int before = a.ws_seq[s];
  const int after = a.ws_seq[s + 1];
  const int W = a.ws_seq[a.B];
  const int splits = a.ws_seq[a.B + 1];
  const int C = a.ws_seq[a.B + 2];
  const bool layout_ok = a.ws_seq[a.B + 3] == a.B && splits >= 1 && (C == 1 || C == 2 || C == 4) &&
                         a.Hkv % C == 0 && splits >= C &&
                         header_bytes(a.B) + acc_bytes(splits, a.G, D) + ml_bytes(splits, a.G) <= a.ws_bytes;
  // A workspace no split pass over these sequences wrote is not followed (every piece index
  // below then stays inside it): the heads of this wave read NaN instead, so the mistake
  // shows in the output rather than passing as a plausible result.
  if (!layout_ok || before < 0 || after < before || W < after ||
      int64_t(W) > int64_t(a.B) * (a.Hkv / C) * unit_span(a.max_blocks, kBlockW)) {
    if (wv == 0 && head_ok) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if constexpr (KV == PKV_F32) static_cast<float*>(a.out)[orow + e] = __builtin_nanf("");
        else static_cast<uint16_t*>(a.out)[orow + e] = 0x7FC0u;
      }
    }
    return;
  }
  const float* ws_acc = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.ws_seq) + header_bytes(a.B));
  const float* ws_ml = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ws_acc) +
                                                      acc_bytes(splits, a.G, D));
  const int span = (after - before) / (a.Hkv / C);            // weighted positions per unit
  const int nb = span > kUnitW ? (span - kUnitW) / kBlockW : 0;
  auto write = [&](const float* v, float inv) {
    if (!head_ok) return;
    if constexpr (KV == PKV_F32) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + e) =
            make_float4(v[e] * inv, v[e + 1] * inv, v[e + 2] * inv, v[e + 3] * inv);
    } else {
      uint32_t w[EPL / 2];
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) w[e] = pack_bf16x2(v[2 * e] * inv, v[2 * e + 1] * inv);
      if constexpr (EPL == 8)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + orow) = make_uint4(w[0], w[1], w[2], w[3]);
      else
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow) = make_uint2(w[0], w[1]);
    }
  };
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  if (nb == 0) {
    if (wv == 0) write(num, 0.f);
    return;
  }
  const int nshare = list_shares(splits / C, W, kBlockW);
  const int sub = g % C;
  const int off = before + (g / C) * span;
  // The shares holding the unit's first and last blocks (a block goes to the share of its
  // first weighted position).
  const int64_t wf = share_of(off + kUnitW, W, nshare), wl = share_of(off + kUnitW + (nb - 1) * kBlockW, W, nshare);
  if (wf == wl) return;
  const int np = int(wl - wf + 1);
  // Share w's pieces of kv head g are those of its wave C*w + g%C.  The unit's piece in
  // share wf is that share's first segment (slot 0) only if the share begins within the
  // unit's weight; in every later share it is the first segment.
  const int64_t piece0 = (wf * C + sub) * 2 + (share_begin(wf, W, nshare) >= off ? 0 : 1);
  // This wave's pieces: [jb, je).
  const int jb = wv * np / MW, je = (wv + 1) * np / MW;

  auto load = [&](int j0, float2* ml, float4 (*x)[EPL / 4]) {
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const int j = std::min(j0 + t, je - 1);
      const int64_t pc = j == 0 ? piece0 : ((wf + j) * C + sub) * 2;
      const int64_t r = pc * a.G + h;
      ml[t] = *reinterpret_cast<const float2*>(ws_ml + r * 2);
      const float4* px = reinterpret_cast<const float4*>(ws_acc + r * D + d0);
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) x[t][i] = px[i];
    }
  };
  float M = -INFINITY, den = 0.f;
  auto fold = [&](int j0, const float2* ml, const float4 (*x)[EPL / 4]) {
    float mb = M;
#pragma unroll
    for (int t = 0; t < BATCH; ++t)
      if (j0 + t < je) mb = fmaxf(mb, ml[t].x);
    const float alpha = __builtin_amdgcn_exp2f(M - mb);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] *= alpha;
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const float c = j0 + t < je ? __builtin_amdgcn_exp2f(ml[t].x - mb) : 0.f;
      den += ml[t].y * c;
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        num[4 * i + 0] += x[t][i].x * c;
        num[4 * i + 1] += x[t][i].y * c;
        num[4 * i + 2] += x[t][i].z * c;
        num[4 * i + 3] += x[t][i].w * c;
      }
    }
    M = mb;
  };
  float2 mlA[BATCH], mlB[BATCH];
  float4 xA[BATCH][EPL / 4], xB[BATCH][EPL / 4];
  if (jb < je) {
    load(jb, mlA, xA);
    for (int j0 = jb; j0 < je; j0 += 2 * BATCH) {
      if (j0 + BATCH < je) load(j0 + BATCH, mlB, xB);
      fold(j0, mlA, xA);
      if (j0 + BATCH >= je) break;
      if (j0 + 2 * BATCH < je) load(j0 + 2 * BATCH, mlA, xA);
      fold(j0 + BATCH, mlB, xB);
    }
  }
  if constexpr (MW == 1) {
    write(num, a.v_scale / den);
    return;
  }
  // The waves' running states (max, sum, accumulator) meet in LDS; wave 0 folds them with
  // the same rule and writes the head.  A wave with no pieces holds (-inf, 0, 0).
  s_md[wv][lane] = make_float2(M, den);
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_num[wv][e][lane] = num[e];
  __syncthreads();
  if (wv != 0) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < MW; ++w) Mx = fmaxf(Mx, s_md[w][lane].x);
  float dsum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < MW; ++w) {
    const float2 md = s_md[w][lane];
    const float c = md.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(md.x - Mx);
    dsum += md.y * c;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += s_num[w][e][lane] * c;
  }
  write(acc, a.v_scale / dsum);
}

// Merge of the split pass with prefix groups: one wave per (four query heads, kv head,
// sequence).  A head's result is spread over the group pass's pieces of its column (member
// s - f of chunk f: the (f, kv head) slot if one share finished the chunk's unit, else the
// pieces of the shares it spans) and over its own unit's pieces (the (s, kv head) slot, or
// the shares' pieces); all of them are folded with the running-softmax rule, eight at a time.
// A piece whose column saw no token (max -inf) adds nothing.  Units the split pass finished
// without a group part were written to `out` there; sequences without tokens get zeros.
template <int KV, int D, int BS>
__global__ __launch_bounds__(64) void paged_attention_grouped_merge_kernel(DecodeArgs a) {
  constexpr int EPL = D / 16;
  constexpr int BATCH = 8;
  const int lane = threadIdx.x & 63;
  const int hq_per_g = (a.G + kMergeHeads - 1) / kMergeHeads;
  const int g = blockIdx.x / hq_per_g, s = blockIdx.y;
  const int h_raw = (blockIdx.x % hq_per_g) * kMergeHeads + (lane >> 4);
  const bool head_ok = h_raw < a.G;
  const int h = head_ok ? h_raw : a.G - 1;
  const int d0 = (lane & 15) * EPL;
  const int64_t orow = ((int64_t(s) * a.Hkv + g) * a.G + h) * D + d0;
  const int C = a.coop, sub = g % C, hg = g / C;
  const int* goff = a.ws_seq + a.B + 4;
  const int Wm = a.ws_seq[a.B], Wg = goff[a.B], nsg = a.ws_seq[2 * a.B + 5];
  int S = 0, nsg_again = 0;   // the split pass's share counts, from the same arguments
  grouped_shares(a, Wm, Wg, S, nsg_again);
  const int nsm = S - nsg;

  // s's group blocks, member blocks, chunk, the chunk's blocks and both offsets: from the
  // split pass's record when it scanned the lists in LDS, else from their definitions.
  int skip, nbm, f = 0, P = 0, moff, goff_f = 0;
  if (a.B <= kScanSeqs) {
    const int4 r0 = *reinterpret_cast<const int4*>(a.ws_rec + 8 * s);
    const int4 r1 = *reinterpret_cast<const int4*>(a.ws_rec + 8 * s + 4);
    moff = r0.x;
    goff_f = r0.y;
    P = r0.z;
    skip = r0.w;
    nbm = r1.x;
    f = r1.y;
  } else {
    skip = group_skip(a, s, BS);
    nbm = seq_blocks(a, s, BS) - skip;
    moff = a.ws_seq[s];
    if (skip > 0) {
      f = a.chunk_first[s];
      P = chunk_blocks(a, f, BS);
      goff_f = goff[f];
    }
  }
  // Group pieces [0, ng) and member pieces [ng, ng + nm): where each lies.
  int ng = 0, nm = 0;
  int64_t g_first = 0, g_wf = 0, m_first = 0, m_wf = 0;
  bool g_slot = false, m_slot = false;
  int col = 0;
  if (skip > 0) {
    col = (s - f) * a.G + h;
    const int off = goff_f + hg * unit_span(P, kGroupBlockW);
    const int64_t wf = share_of(off + kUnitW, Wg, nsg), wl = share_of(off + kUnitW + (P - 1) * kGroupBlockW, Wg, nsg);
    g_slot = wf == wl;
    ng = g_slot ? 1 : int(wl - wf + 1);
    g_wf = wf;
    g_first = (wf * C + sub) * 2 + (share_begin(wf, Wg, nsg) >= off ? 0 : 1);
  }
  if (nbm > 0) {
    const int off = moff + hg * unit_span(nbm, kBlockW);
    const int64_t wf = share_of(off + kUnitW, Wm, nsm), wl = share_of(off + kUnitW + (nbm - 1) * kBlockW, Wm, nsm);
    if (wf == wl && skip == 0) return;   // finished and written by the split pass
    m_slot = wf == wl;
    nm = m_slot ? 1 : int(wl - wf + 1);
    m_wf = wf;
    m_first = (wf * C + sub) * 2 + (share_begin(wf, Wm, nsm) >= off ? 0 : 1);
  }
  auto row_of = [&](int j, const float*& acc, const float*& ml) {
    int64_t r;
    if (j < ng) {
      const int64_t pc = j == 0 ? g_first : ((g_wf + j) * C + sub) * 2;
      if (g_slot) {
        r = (int64_t(f) * a.Hkv + g) * kGroupCols + col;
        acc = a.ws_fgacc; ml = a.ws_fgml;
      } else {
        r = pc * kGroupCols + col;
        acc = a.ws_gacc; ml = a.ws_gml;
      }
    } else {
      const int jm = j - ng;
      const int64_t pc = jm == 0 ? m_first : ((m_wf + jm) * C + sub) * 2;
      if (m_slot) {
        r = (int64_t(s) * a.Hkv + g) * a.G + h;
        acc = a.ws_macc; ml = a.ws_mml;
      } else {
        r = pc * a.G + h;
        acc = a.ws_acc; ml = a.ws_ml;
      }
    }
    acc += r * D + d0;
    ml += r * 2;
  };
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  float M = -INFINITY, den = 0.f;
  const int np = ng + nm;
  for (int j0 = 0; j0 < np; j0 += BATCH) {
    float2 ml[BATCH];
    float4 x[BATCH][EPL / 4];
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const float* pa;
      const float* pm;
      row_of(std::min(j0 + t, np - 1), pa, pm);
      ml[t] = *reinterpret_cast<const float2*>(pm);
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) x[t][i] = reinterpret_cast<const float4*>(pa)[i];
    }
    float mb = M;
#pragma unroll
    for (int t = 0; t < BATCH; ++t)
      if (j0 + t < np) mb = fmaxf(mb, ml[t].x);
    if (mb == -INFINITY) continue;                  // nothing attended yet
    const float alpha = __builtin_amdgcn_exp2f(M - mb);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] *= alpha;
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const float c = j0 + t < np ? __builtin_amdgcn_exp2f(ml[t].x - mb) : 0.f;   // 0 for a -inf piece
      den += ml[t].y * c;
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        num[4 * i + 0] += x[t][i].x * c;
        num[4 * i + 1] += x[t][i].y * c;
        num[4 * i + 2] += x[t][i].z * c;
        num[4 * i + 3] += x[t][i].w * c;
      }
    }
    M = mb;
  }
  if (!head_ok) return;
  const float inv = den > 0.f ? a.v_scale / den : 0.f;
  if constexpr (KV == PKV_F32) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + e) =
          make_float4(num[e] * inv, num[e + 1] * inv, num[e + 2] * inv, num[e + 3] * inv);
  } else {
    uint32_t w[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) w[e] = pack_bf16x2(num[2 * e] * inv, num[2 * e + 1] * inv);
    if constexpr (EPL == 8)
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + orow) = make_uint4(w[0], w[1], w[2], w[3]);
    else
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow) = make_uint2(w[0], w[1]);
  }
}

// ---- host side --------------------------------------------------------------------------

// Sub-tiles per loop iteration: about 4 KiB of K (and as much V) per wave per step.
template <int KV, int D>
constexpr int subtiles_per_step() {
  constexpr int sub_bytes = 16 * D * KvTraits<KV>::EB;
  return sub_bytes >= 4096 ? 1 : 4096 / sub_bytes;
}

using KernelFn = void (*)(DecodeArgs);

struct KernelPair {
  // Index [mixed]: 0 streams all K/V with the non-temporal hint, 1 reads the leading
  // blocks that a sequence shares through the caches.
  KernelFn split[2];         // plain decode
  KernelFn split_append[2];  // decode step that stores each sequence's appended token first
  KernelFn split_contig;     // plain decode over contiguous per-sequence placement
  KernelFn grouped[2];       // [append]: split pass with prefix groups read once per chunk
  KernelFn grouped_merge;
  KernelFn merge;            // one wave per (sequence, kv head, four query heads)
  KernelFn merge_long;       // kMergeWavesLong waves each, for units that span many shares
};

template <int KV, int D, int BS>
KernelPair kernels_for() {
  constexpr int N = subtiles_per_step<KV, D>();
  // The f32, D 128 decode step has no registers to spare for the per-sequence policy (it
  // would spill), so it always streams.
  constexpr bool kMix = !(KV == PKV_F32 && D == 128);
  return {{paged_attention_split_kernel<KV, D, BS, N, false, false>,
           paged_attention_split_kernel<KV, D, BS, N, false, true>},
          {paged_attention_split_kernel<KV, D, BS, N, true, false>,
           paged_attention_split_kernel<KV, D, BS, N, true, kMix>},
          paged_attention_split_kernel<KV, D, BS, N, false, false, true>,
          {paged_attention_grouped_kernel<KV, D, BS, N, false>, paged_attention_grouped_kernel<KV, D, BS, N, true>},
          paged_attention_grouped_merge_kernel<KV, D, BS>,
          paged_attention_merge_kernel<KV, D, BS, 1>,
          paged_attention_merge_kernel<KV, D, BS, kMergeWavesLong>};
}

bool pick_kernels(pkv_dtype kv, int D, int bs, KernelPair* kp) {
#define PKV_CASE(KVT, DD, BB) \
  if (kv == KVT && D == DD && bs == BB) { *kp = kernels_for<KVT, DD, BB>(); return true; }
  PKV_CASE(PKV_F32, 64, 16) PKV_CASE(PKV_F32, 64, 32) PKV_CASE(PKV_F32, 128, 16) PKV_CASE(PKV_F32, 128, 32)
  PKV_CASE(PKV_BF16, 64, 16) PKV_CASE(PKV_BF16, 64, 32) PKV_CASE(PKV_BF16, 128, 16) PKV_CASE(PKV_BF16, 128, 32)
  PKV_CASE(PKV_FP8_E4M3FN, 64, 16) PKV_CASE(PKV_FP8_E4M3FN, 64, 32)
  PKV_CASE(PKV_FP8_E4M3FN, 128, 16) PKV_CASE(PKV_FP8_E4M3FN, 128, 32)
#undef PKV_CASE
  return false;
}

// Workgroups of the split kernel one CU keeps resident, and the CU count (cached per
// device and kernel).
pkv_status resident_wgs(KernelFn fn, int* per_cu_out, int* cus_out) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, std::pair<int, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "hipGetDevice failed");
  const uint64_t key = (uint64_t(reinterpret_cast<uintptr_t>(fn)) << 8) ^ uint64_t(dev);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *per_cu_out = it->second.first;
      *cus_out = it->second.second;
      return PKV_OK;
    }
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return pkv::fail(PKV_HIP_ERROR, "hipDeviceGetAttribute(multiprocessor count) failed");
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                   kWavesPerWG * 64, 0) != hipSuccess)
    return pkv::fail(PKV_HIP_ERROR, "hipOccupancyMaxActiveBlocksPerMultiprocessor failed");
  per_cu = std::max(1, per_cu);
  cus = std::max(1, cus);
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = {per_cu, cus};
  *per_cu_out = per_cu;
  *cus_out = cus;
  return PKV_OK;
}

int elem_bytes(pkv_dtype t) { return t == PKV_F32 ? 4 : t == PKV_BF16 ? 2 : t == PKV_FP8_E4M3FN ? 1 : 0; }

pkv_status check_shape(const char* fn, int B, int Hq, int Hkv, int D, int bs, pkv_dtype qd,
                       pkv_dtype kd) {
  if (B < 0 || Hq <= 0 || Hkv <= 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_seqs=%d num_q_heads=%d num_kv_heads=%d", fn, B, Hq, Hkv);
  if (Hq % Hkv != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", fn, Hq, Hkv);
  if (Hq / Hkv > kMaxGroup)
    return pkv::fail(PKV_UNSUPPORTED, "%s: group size %d > %d", fn, Hq / Hkv, kMaxGroup);
  const bool types_ok = (qd == PKV_F32 && kd == PKV_F32) || (qd == PKV_BF16 && kd == PKV_BF16) ||
                        (qd == PKV_BF16 && kd == PKV_FP8_E4M3FN);
  if (!types_ok) return pkv::fail(PKV_UNSUPPORTED, "%s: q_dtype=%d kv_dtype=%d", fn, int(qd), int(kd));
  KernelPair kp;
  if (!pick_kernels(kd, D, bs, &kp))
    return pkv::fail(PKV_UNSUPPORTED, "%s: head_dim=%d block_size=%d", fn, D, bs);
  return PKV_OK;
}

// Default split count of a kernel variant: one share per wave of `target` waves per CU,
// capped by what the plain and the appending split kernels can keep resident (the lower of
// the two, so that both entry points launch the same shares).  Measured on MI355X: f32 /
// bf16 caches stream best with 8 waves (2 per SIMD) per CU, fp8 caches, with more
// arithmetic per byte, with 16 where registers allow it.  The count depends on neither the
// load policy nor shared_prefix_blocks, so the output bits do not either.
pkv_status default_splits(const KernelPair& kp, pkv_dtype kv, int* splits) {
  int a = 0, b = 0, cus = 0;
  pkv_status st = resident_wgs(kp.split[0], &a, &cus);
  if (st != PKV_OK) return st;
  if ((st = resident_wgs(kp.split_append[0], &b, &cus)) != PKV_OK) return st;
  const int target_wgs = (kv == PKV_FP8_E4M3FN ? 16 : 8) / kWavesPerWG;
  *splits = cus * std::max(1, std::min(target_wgs, std::min(a, b))) * kWavesPerWG;
  return PKV_OK;
}

pkv_status effective_splits(const KernelPair& kp, pkv_dtype kv, int requested, int* splits) {
  if (requested < 0) return pkv::fail(PKV_INVALID_ARG, "num_splits=%d must be >= 0", requested);
  if (requested > 0) {
    *splits = requested;
    return PKV_OK;
  }
  return default_splits(kp, kv, splits);
}

size_t workspace_bytes_for(int splits, int B, int G, int D) {
  return size_t(header_bytes(B) + acc_bytes(splits, G, D) + ml_bytes(splits, G));
}

// Workspace of the split pass with prefix groups, in order: a header (member and group work
// offsets and the record), the member pieces of shares (as without groups), member units
// finished inside a share [B * Hkv][G], the group pieces of shares [splits * 2][32], group
// units finished inside a share [B * Hkv][32]; accumulators float32 [D] and (max, sum) pairs.
struct GroupedLayout {
  int64_t hdr, sacc, sml, macc, mml, gacc, gml, fgacc, fgml, rec;
  int64_t total() const { return hdr + sacc + sml + macc + mml + gacc + gml + fgacc + fgml + rec; }
};

GroupedLayout grouped_layout(int splits, int B, int Hkv, int G, int D) {
  GroupedLayout l;
  l.hdr = round256((2 * int64_t(B) + 8) * 4);
  l.sacc = acc_bytes(splits, G, D);
  l.sml = ml_bytes(splits, G);
  l.macc = round256(int64_t(B) * Hkv * G * D * 4);
  l.mml = round256(int64_t(B) * Hkv * G * 2 * 4);
  l.gacc = round256(int64_t(splits) * 2 * kGroupCols * D * 4);
  l.gml = round256(int64_t(splits) * 2 * kGroupCols * 2 * 4);
  l.fgacc = round256(int64_t(B) * Hkv * kGroupCols * D * 4);
  l.fgml = round256(int64_t(B) * Hkv * kGroupCols * 2 * 4);
  l.rec = round256(int64_t(B) * 8 * 4);
  return l;
}

// Split count of the grouped pass: as requested, at least two (one share of each kind).
int grouped_splits(int splits, int B, int Hkv, int max_blocks) {
  return int(std::max<int64_t>(2, std::min<int64_t>(splits, 2 * int64_t(B) * Hkv * std::max(1, max_blocks))));
}

enum Phase { kBoth, kSplitOnly, kMergeOnly };

// k_new / v_new non-null: the decode step with append (the split pass stores each
// sequence's token at position L-1 from k_new / v_new into the writable caches).
pkv_status run_decode(const char* fn, Phase phase, void* out, const void* q, const void* k_new,
                      const void* v_new, const void* k_cache, const void* v_cache,
                      void* k_cache_w, void* v_cache_w, const int32_t* block_tables,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int D, int bs,
                      int num_blocks, int max_blocks, float scale, float k_scale, float v_scale,
                      pkv_dtype qd, pkv_dtype kd, int num_splits, void* workspace,
                      size_t workspace_bytes, const int32_t* shared_prefix, void* stream,
                      const int32_t* seq_first_block = nullptr, const int32_t* chunk_first = nullptr,
                      const int32_t* chunk_src = nullptr, const int32_t* group_blocks = nullptr) {
  const bool append = k_new != nullptr || v_new != nullptr;
  const bool contig = seq_first_block != nullptr;
  const bool grouped = chunk_first != nullptr || chunk_src != nullptr || group_blocks != nullptr;
  pkv_status st = check_shape(fn, B, Hq, Hkv, D, bs, qd, kd);
  if (st != PKV_OK) return st;
  if (num_blocks <= 0 || max_blocks < 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_blocks=%d max_blocks_per_seq=%d", fn, num_blocks, max_blocks);
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f) || scale == INFINITY ||
      k_scale == INFINITY || v_scale == INFINITY)
    return pkv::fail(PKV_INVALID_ARG, "%s: scales must be positive and finite", fn);
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (!contig && max_blocks > 0 && !block_tables))
    return pkv::fail(PKV_INVALID_ARG, "%s: null pointer", fn);
  if (contig && (append || shared_prefix))
    return pkv::fail(PKV_INVALID_ARG, "%s: the contiguous placement takes no append or shared-prefix counts", fn);
  if (reinterpret_cast<uintptr_t>(seq_first_block) % 4 != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: seq_first_block must be 4-byte aligned", fn);
  if (grouped && (!chunk_first || !chunk_src || !group_blocks))
    return pkv::fail(PKV_INVALID_ARG, "%s: chunk_first, chunk_src and group_blocks must all be given", fn);
  if (grouped && (contig || shared_prefix || phase != kBoth))
    return pkv::fail(PKV_INVALID_ARG, "%s: prefix groups take no contiguous placement or shared-prefix counts", fn);
  if ((reinterpret_cast<uintptr_t>(chunk_first) | reinterpret_cast<uintptr_t>(chunk_src) |
       reinterpret_cast<uintptr_t>(group_blocks)) % 4 != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: chunk_first, chunk_src and group_blocks must be 4-byte aligned", fn);
  if (append && (!k_new || !v_new || !k_cache_w || !v_cache_w))
    return pkv::fail(PKV_INVALID_ARG, "%s: k_new and v_new must both be given", fn);
  if (!pkv::aligned16({out, q, k_cache, v_cache, k_new, v_new, workspace}))
    return pkv::fail(PKV_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(shared_prefix) % 4 != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: shared_prefix_blocks must be 4-byte aligned", fn);
  KernelPair kp;
  pick_kernels(kd, D, bs, &kp);
  int splits = 0;
  if ((st = effective_splits(kp, kd, num_splits, &splits)) != PKV_OK) return st;
  const int G = Hq / Hkv;
  // The reduce pass takes the partials' layout from the header the split pass wrote, so it
  // needs only the header to be addressable; the merge kernel checks the rest on the device.
  const size_t need = grouped ? size_t(grouped_layout(grouped_splits(splits, B, Hkv, max_blocks), B, Hkv, G, D).total())
                      : phase == kMergeOnly ? size_t(header_bytes(B))
                                            : workspace_bytes_for(splits, B, G, D);
  if (!workspace || workspace_bytes < need)
    return pkv::fail(PKV_INVALID_ARG, "%s: workspace of %zu bytes < %zu required", fn,
                     workspace_bytes, need);
  if (int64_t(B) > 65535 || Hkv > 65535)
    return pkv::fail(PKV_UNSUPPORTED, "%s: num_seqs and num_kv_heads must be <= 65535", fn);
  if (int64_t(B) * Hkv * (int64_t(max_blocks) * kGroupBlockW + kUnitW) * (grouped ? 2 : 1) > int64_t(INT32_MAX))
    return pkv::fail(PKV_UNSUPPORTED, "%s: num_seqs * max_blocks_per_seq * num_kv_heads is too large for the work list",
                     fn);

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.B = B;
  a.Hkv = Hkv;
  a.G = G;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  // More shares than (sequence, kv head, block) triples would only launch idle waves; the
  // table width bounds the triples without reading the device-side lengths (with prefix
  // groups, twice: group and member lists; and at least one share of each kind).
  a.splits = grouped ? grouped_splits(splits, B, Hkv, max_blocks)
                     : int(std::max<int64_t>(1, std::min<int64_t>(splits, int64_t(B) * Hkv * max_blocks)));
  // The partials are laid out for the share count the kernels use, which the split pass
  // records in the header and the merge reads back.
  a.ws_seq = static_cast<int*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + header_bytes(B));
  a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.ws_acc) + acc_bytes(a.splits, G, D));
  a.ws_bytes = int64_t(workspace_bytes);
  a.coop = 1;
  // With prefix groups every head group must leave at least two shares (one of each kind).
  const int coop_min_shares = grouped ? 4 : 2;
  while (a.coop < kWavesPerWG && Hkv % (2 * a.coop) == 0 && a.splits >= coop_min_shares * a.coop) a.coop *= 2;
  a.qk_scale_log2 = scale * k_scale * kLog2e;
  a.v_scale = v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache_w = static_cast<uint8_t*>(k_cache_w);
  a.v_cache_w = static_cast<uint8_t*>(v_cache_w);
  a.k_inv = 1.0f / k_scale;
  a.v_inv = 1.0f / v_scale;
  a.shared_prefix = shared_prefix;
  a.seq_first_block = seq_first_block;
  a.chunk_first = chunk_first;
  a.chunk_src = chunk_src;
  a.group_blocks = group_blocks;
  a.appending = append ? 1 : 0;
  if (grouped) {
    // Grouped layout: the member share pieces sit where the plain layout puts its pieces.
    const GroupedLayout l = grouped_layout(a.splits, B, Hkv, G, D);
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.ws_seq = reinterpret_cast<int*>(w);
    a.ws_acc = reinterpret_cast<float*>(w + l.hdr);
    a.ws_ml = reinterpret_cast<float*>(w + l.hdr + l.sacc);
    a.ws_macc = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml);
    a.ws_mml = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml + l.macc);
    a.ws_gacc = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml + l.macc + l.mml);
    a.ws_gml = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml + l.macc + l.mml + l.gacc);
    a.ws_fgacc = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml + l.macc + l.mml + l.gacc + l.gml);
    a.ws_fgml = reinterpret_cast<float*>(w + l.hdr + l.sacc + l.sml + l.macc + l.mml + l.gacc + l.gml + l.fgacc);
    a.ws_rec = reinterpret_cast<int*>(w + l.hdr + l.sacc + l.sml + l.macc + l.mml + l.gacc + l.gml + l.fgacc + l.fgml);
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (phase != kMergeOnly) {
    const unsigned wgs = unsigned((int64_t(a.splits) + kWavesPerWG - 1) / kWavesPerWG);
    const int mixed = shared_prefix != nullptr ? 1 : 0;
    KernelFn kfn = grouped  ? kp.grouped[append ? 1 : 0]
                   : contig ? kp.split_contig
                   : append ? kp.split_append[mixed]
                            : kp.split[mixed];
    void *ev0 = nullptr, *ev1 = nullptr;
    if (pkv::take_launch_events(&ev0, &ev1)) {
      // The dispatch itself records the events, so they time the kernel alone.
      void* kargs[] = {&a};
      hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kfn), dim3(wgs),
                                        dim3(kWavesPerWG * 64), kargs, 0, hs,
                                        static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0);
      if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: split launch: %s", fn, hipGetErrorString(e));
    } else {
      hipLaunchKernelGGL(kfn, dim3(wgs), dim3(kWavesPerWG * 64), 0, hs, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: split launch: %s", fn, hipGetErrorString(e));
  }
  if (phase != kSplitOnly) {
    const unsigned merge_x = unsigned(Hkv * ((G + kMergeHeads - 1) / kMergeHeads));
    // Units span about (shares) / (units) shares each, where the table width bounds the
    // work list: many (long contexts) take the merge whose waves split a unit's pieces; a
    // few take one wave per unit.
    const int64_t units = int64_t(B) * (Hkv / a.coop);
    const int64_t shares = std::min<int64_t>(a.splits / a.coop, units * max_blocks);
    const bool long_units = shares >= int64_t(kLongMergePieces) * units;
    if (grouped)
      hipLaunchKernelGGL(kp.grouped_merge, dim3(merge_x, unsigned(B)), dim3(64), 0, hs, a);
    else if (long_units)
      hipLaunchKernelGGL(kp.merge_long, dim3(merge_x, unsigned(B)), dim3(64 * kMergeWavesLong), 0, hs, a);
    else
      hipLaunchKernelGGL(kp.merge, dim3(merge_x, unsigned(B)), dim3(64), 0, hs, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: merge launch: %s", fn, hipGetErrorString(e));
  }
  return PKV_OK;
}

// Scratch of the entry point that allocates nothing: the workspace of
// pkv_paged_attention_decode_noalloc lives in this file-scope array, one copy per device,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not the
// device copy, so kernels are handed the address hipGetSymbolAddress reports for the
// current device (resolved on the first call on each device and kept).
constexpr size_t kScratchBytes = size_t(48) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

pkv_status scratch_address(void** ptr_out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return pkv::fail(PKV_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pkv::fail(PKV_HIP_ERROR, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    ptr[dev] = p;
  }
  *ptr_out = ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                              int block_size, int num_blocks, int max_blocks_per_seq,
                                              float scale, float k_scale, float v_scale, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int num_splits,
                                              const int32_t* shared_prefix_blocks, void* stream) {
  const char* fn = "pkv_paged_attention_decode_noalloc";
  pkv_status st = check_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, q_dtype, kv_dtype);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  KernelPair kp;
  pick_kernels(kv_dtype, head_dim, block_size, &kp);
  int splits = 0;
  if ((st = effective_splits(kp, kv_dtype, num_splits, &splits)) != PKV_OK) return st;
  const size_t need = workspace_bytes_for(splits, num_seqs, num_q_heads / num_kv_heads, head_dim);
  if (need > kScratchBytes)
    return pkv::fail(PKV_INVALID_ARG,
                     "%s: the call needs %zu bytes of scratch, more than the %zu-byte maximum; pass a smaller "
                     "num_splits or use pkv_paged_attention_decode with a workspace",
                     fn, need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != PKV_OK) return st;
  return run_decode(fn, kBoth, out, q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_tables,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                    max_blocks_per_seq, scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits, ws, kScratchBytes,
                    shared_prefix_blocks, stream);
}

pkv_status pkv_paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                              int head_dim, int block_size, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int num_splits, size_t* bytes) {
  pkv_status st = check_shape("pkv_paged_attention_workspace_size", num_seqs, num_q_heads,
                              num_kv_heads, head_dim, block_size, q_dtype, kv_dtype);
  if (st != PKV_OK) return st;
  if (!bytes) return pkv::fail(PKV_INVALID_ARG, "pkv_paged_attention_workspace_size: null output");
  KernelPair kp;
  pick_kernels(kv_dtype, head_dim, block_size, &kp);
  int splits = 0;
  if ((st = effective_splits(kp, kv_dtype, num_splits, &splits)) != PKV_OK) return st;
  *bytes = workspace_bytes_for(splits, num_seqs, num_q_heads / num_kv_heads, head_dim);
  return PKV_OK;
}

pkv_status pkv_paged_attention_default_splits(int head_dim, int block_size, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int* splits) {
  pkv_status st = check_shape("pkv_paged_attention_default_splits", 1, 1, 1, head_dim, block_size,
                              q_dtype, kv_dtype);
  if (st != PKV_OK) return st;
  if (!splits) return pkv::fail(PKV_INVALID_ARG, "pkv_paged_attention_default_splits: null output");
  KernelPair kp;
  pick_kernels(kv_dtype, head_dim, block_size, &kp);
  return default_splits(kp, kv_dtype, splits);
}

#define PKV_DECODE_PARAMS                                                                        \
  void *out, const void *q, const void *k_cache, const void *v_cache,                           \
      const int32_t *block_tables, const int32_t *context_lens, int num_seqs, int num_q_heads,  \
      int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,   \
      float scale, float k_scale, float v_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,          \
      int num_splits, void *workspace, size_t workspace_bytes, const int32_t *shared_prefix_blocks, \
      void *stream
#define PKV_DECODE_ARGS                                                                          \
  out, q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,     \
      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, \
      scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits, workspace, workspace_bytes,        \
      shared_prefix_blocks, stream

pkv_status pkv_paged_attention_decode(PKV_DECODE_PARAMS) {
  return run_decode("pkv_paged_attention_decode", kBoth, PKV_DECODE_ARGS);
}
pkv_status pkv_paged_attention_split(PKV_DECODE_PARAMS) {
  return run_decode("pkv_paged_attention_split", kSplitOnly, PKV_DECODE_ARGS);
}
pkv_status pkv_paged_attention_reduce(PKV_DECODE_PARAMS) {
  return run_decode("pkv_paged_attention_reduce", kMergeOnly, PKV_DECODE_ARGS);
}

pkv_status pkv_contiguous_attention_decode(void* out, const void* q, const void* k_base, const void* v_base,
                                           const int32_t* seq_first_block, const int32_t* context_lens,
                                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                           int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                                           float k_scale, float v_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                           int num_splits, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (num_seqs > 0 && !seq_first_block)
    return pkv::fail(PKV_INVALID_ARG, "pkv_contiguous_attention_decode: null seq_first_block");
  return run_decode("pkv_contiguous_attention_decode", kBoth, out, q, nullptr, nullptr, k_base, v_base, nullptr,
                    nullptr, nullptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, max_blocks_per_seq, scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits,
                    workspace, workspace_bytes, nullptr, stream, seq_first_block);
}

#define PKV_STEP_PARAMS                                                                          \
  void *out, const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache, \
      const int32_t *block_tables, const int32_t *context_lens, int num_seqs, int num_q_heads,  \
      int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,   \
      float scale, float k_scale, float v_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,          \
      int num_splits, void *workspace, size_t workspace_bytes, const int32_t *shared_prefix_blocks, \
      void *stream
#define PKV_STEP_ARGS                                                                            \
  out, q, k_new, v_new, k_cache, v_cache, k_cache, v_cache, block_tables, context_lens,         \
      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, \
      scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits, workspace, workspace_bytes,        \
      shared_prefix_blocks, stream

pkv_status pkv_paged_decode_step(PKV_STEP_PARAMS) {
  if (!k_new || !v_new) return pkv::fail(PKV_INVALID_ARG, "pkv_paged_decode_step: null k_new / v_new");
  return run_decode("pkv_paged_decode_step", kBoth, PKV_STEP_ARGS);
}
pkv_status pkv_paged_attention_grouped_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                                      int block_size, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                                      int num_splits, int max_blocks_per_seq, size_t* bytes) {
  pkv_status st = check_shape("pkv_paged_attention_grouped_workspace_size", num_seqs, num_q_heads, num_kv_heads,
                              head_dim, block_size, q_dtype, kv_dtype);
  if (st != PKV_OK) return st;
  if (!bytes || max_blocks_per_seq < 0)
    return pkv::fail(PKV_INVALID_ARG, "pkv_paged_attention_grouped_workspace_size: bad arguments");
  KernelPair kp;
  pick_kernels(kv_dtype, head_dim, block_size, &kp);
  int splits = 0;
  if ((st = effective_splits(kp, kv_dtype, num_splits, &splits)) != PKV_OK) return st;
  *bytes = size_t(grouped_layout(grouped_splits(splits, num_seqs, num_kv_heads, max_blocks_per_seq), num_seqs,
                                 num_kv_heads, num_q_heads / num_kv_heads, head_dim)
                      .total());
  return PKV_OK;
}

pkv_status pkv_paged_attention_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              const int32_t* chunk_first, const int32_t* chunk_src,
                                              const int32_t* group_blocks, int num_seqs, int num_q_heads,
                                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                              int max_blocks_per_seq, float scale, float k_scale, float v_scale,
                                              pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode_grouped";
  if (num_seqs > 0 && (!chunk_first || !chunk_src || !group_blocks))
    return pkv::fail(PKV_INVALID_ARG, "%s: null chunk_first / chunk_src / group_blocks", fn);
  return run_decode(fn, kBoth, out, q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_tables,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                    max_blocks_per_seq, scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits, workspace,
                    workspace_bytes, nullptr, stream, nullptr, chunk_first, chunk_src, group_blocks);
}

pkv_status pkv_paged_decode_step_grouped(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                         const int32_t* chunk_first, const int32_t* chunk_src,
                                         const int32_t* group_blocks, int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                         float scale, float k_scale, float v_scale, pkv_dtype q_dtype,
                                         pkv_dtype kv_dtype, int num_splits, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  const char* fn = "pkv_paged_decode_step_grouped";
  if (!k_new || !v_new) return pkv::fail(PKV_INVALID_ARG, "%s: null k_new / v_new", fn);
  if (num_seqs > 0 && (!chunk_first || !chunk_src || !group_blocks))
    return pkv::fail(PKV_INVALID_ARG, "%s: null chunk_first / chunk_src / group_blocks", fn);
  return run_decode(fn, kBoth, out, q, k_new, v_new, k_cache, v_cache, k_cache, v_cache, block_tables,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                    max_blocks_per_seq, scale, k_scale, v_scale, q_dtype, kv_dtype, num_splits, workspace,
                    workspace_bytes, nullptr, stream, nullptr, chunk_first, chunk_src, group_blocks);
}

pkv_status pkv_paged_decode_step_split(PKV_STEP_PARAMS) {
  if (!k_new || !v_new)
    return pkv::fail(PKV_INVALID_ARG, "pkv_paged_decode_step_split: null k_new / v_new");
  return run_decode("pkv_paged_decode_step_split", kSplitOnly, PKV_STEP_ARGS);
}

}  // extern "C"
