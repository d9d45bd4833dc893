// Multi-query paged attention for gfx950 (MI355X): several query tokens per sequence with a
// causal mask, over the same block tables and pool as decode.  This covers a prefill (every
// token of the prompt is a query), a chunk of a prefill (the last n tokens of a longer
// context) and the check of drafted tokens in speculative decoding.
//
// What is computed:
//  * "What is PagedAttention?" (qubittool glossary), "How It Works: Map Logical to Physical
//    Blocks": a prefill allocates blocks for the whole input, so the prompt's K/V sit in the
//    pool behind the sequence's block table before its attention runs.
//  * "PagedAttention: Optimizing KV Cache in vLLM" (grasp.study), §3 "Making it Work: The
//    PagedAttention Kernel": the kernel walks the blocks in logical order with a running
//    softmax and reaches attention over a contiguous layout; "Conclusion": speculative
//    decoding, where several drafted tokens are checked against the cache in one pass.
//  * Neither page writes out the attention of several query tokens; the reading taken is
//    causal attention: sequence s's n_s queries are its last n_s tokens, and the query at
//    position P = L_s - n_s + i attends to tokens 0..P.  n_s = 1 is decode.
//
// How it maps onto CDNA4
//  * Columns: a column is one (query token, query head) pair of one kv head; a workgroup
//    of 8 waves owns 128*CT consecutive columns of one (sequence, kv head), each wave 16*CT
//    (CT matrix-instruction column tiles).  Every tile re-reads its unit's K/V, so wide
//    tiles keep that traffic down.  With G query heads per kv head the columns of
//    one query token are adjacent, so every K/V byte a workgroup stages serves all of them.
//  * Staging: each step the workgroup copies SUBS 16-token sub-tiles of K and of V (32 KiB
//    for bf16, D 128) from the pool into LDS, one 16-byte chunk per thread per load, with the
//    next step's loads in flight while the current step computes (two LDS buffers, one
//    barrier per step).  The sequence's block-table entries are staged in LDS once, so a
//    chunk's address depends on an LDS read, not on a global load.
//  * Matrix products: the pool layout makes chunk 64*i + lane of a sub-tile exactly lane's
//    operand (attention_tile.h): QK^T with K as the A operand and q (held in registers) as B,
//    then PV with the probabilities reused in place as B.  Each K/V operand read from LDS
//    feeds CT products.
//  * Causal mask and running softmax (base 2): token t is kept for a column iff t <= P of
//    that column; the rest get -inf by select.  A step that lies entirely past a wave's last
//    position is skipped by that wave (it still stages its share of the loads).  V elements
//    of slots at or past L_s are zeroed (an unwritten tail slot may hold NaN).
//  * Order: all tiles of one (sequence, kv head) run on one XCD (sharing its L2), launched
//    last tile first, so the tiles with the most keys start earliest.  Given a workspace, a
//    plan pass first orders each XCD's (sequence, kv head) units longest first.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "attention_tile.h"
#include "status.h"

namespace {

using namespace pkv::tile;

constexpr int kWaves = 8;                   // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kXcds = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kMaxTableBytes = 64 * 1024;   // block-table entries staged in LDS, at most
constexpr int kTblPad = 8;                  // -1 entries after them (a step reads at most 7 past)

// One workgroup slot of the tile path: which query tile of which (sequence, kv head) it
// runs, with that sequence's clamped query range and length, and the steps the tile takes
// (its work).  unit < 0 marks a slot with nothing to do.
struct TileJob {
  int unit, tile, q0, n, L, steps, pad0, pad1;
};

struct PrefillArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int B, Hkv, G, num_blocks, max_blocks, num_q_tokens;
  int tiles;            // query tiles per (sequence, kv head)
  int units_per_xcd;    // ceil(B * Hkv / kXcds)
  int per_xcd;          // units_per_xcd * tiles: workgroup slots per XCD
  int cols;             // (query, head) columns per tile
  int step_tok;         // keys staged per step
  float qk_scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
  int64_t max_tok;      // max_blocks * block size: keys a table can reach
  TileJob* plan;        // launch order, [kXcds][per_xcd], or null for the default order
};

// Sequence s's query range and length, clamped as the kernels read them.
struct SeqSpan {
  int q0, n, L;
};

__device__ __forceinline__ SeqSpan seq_span(const PrefillArgs& a, int s) {
  int q0 = a.query_start[s], q1 = a.query_start[s + 1];
  q0 = std::min(std::max(q0, 0), a.num_q_tokens);
  q1 = std::min(std::max(q1, q0), a.num_q_tokens);
  int L = std::max(a.context_lens[s], 0);
  if (int64_t(L) > a.max_tok) L = int(a.max_tok);
  return SeqSpan{q0, q1 - q0, L};
}

// Query tiles of a unit with at least one query column: min(ceil(n G / cols), tiles).
__device__ __forceinline__ int live_tiles(const PrefillArgs& a, const SeqSpan& sp) {
  return int(std::min<int64_t>((int64_t(sp.n) * a.G + a.cols - 1) / a.cols, a.tiles));
}

// The record of tile `tile` (live) of unit `unit`, with the steps it takes.
__device__ __forceinline__ TileJob make_job(const PrefillArgs& a, int unit, int tile, const SeqSpan& sp) {
  const int col0 = tile * a.cols;
  const int last_q = std::min(sp.n - 1, (col0 + a.cols - 1) / a.G);
  const int ntok = std::max(sp.L - sp.n + last_q + 1, 0);
  return TileJob{unit, tile, sp.q0, sp.n, sp.L, (ntok + a.step_tok - 1) / a.step_tok, 0, 0};
}

// Slot j of XCD xcd in the default order: the (sequence, kv head) units are dealt to the
// XCDs round-robin (unit u on XCD u % kXcds), and every query tile of a unit goes to the
// unit's XCD, so the unit's K/V stays in that XCD's L2 while its tiles run; a unit's tiles
// follow each other, last (longest) tile first.
__device__ __forceinline__ TileJob tile_job(const PrefillArgs& a, int xcd, int j) {
  const int unit = xcd + kXcds * (j / a.tiles);
  const int tile = a.tiles - 1 - j % a.tiles;
  if (unit >= a.B * a.Hkv) return TileJob{-1, 0, 0, 0, 0, 0, 0, 0};
  const SeqSpan sp = seq_span(a, unit / a.Hkv);
  if (tile >= live_tiles(a, sp)) return TileJob{-1, 0, 0, 0, 0, 0, 0, 0};
  return make_job(a, unit, tile, sp);
}

// Sub-tiles staged per step: 16 KiB of K plus 16 KiB of V, at most 8 sub-tiles.
template <int KV, int D>
constexpr int step_subtiles() {
  constexpr int sub = 16 * D * KvTraits<KV>::EB;
  return 16384 / sub > 8 ? 8 : 16384 / sub;
}

template <int KV, int D, int BS, int CT>
__global__ __launch_bounds__(kThreads, 1) void paged_attention_prefill_kernel(PrefillArgs a) {
  // KV is the pool's element type; CKV the type staged in LDS and used by the matrix
  // products.  An fp8 cache is widened to bf16 (exactly) once, while the workgroup stages a
  // step, instead of by each of its waves in every product.
  constexpr int CKV = KV == PKV_FP8_E4M3FN ? PKV_BF16 : KV;
  using F = Frag<CKV, D>;
  using T = KvTraits<CKV>;
  constexpr int X = 16 / T::EB;
  constexpr int SUB_BYTES = 16 * D * T::EB;                 // an LDS sub-tile
  constexpr int SUB_CHUNKS = SUB_BYTES / 16;
  constexpr int SUB_BYTES_P = 16 * D * KvTraits<KV>::EB;    // a pool sub-tile
  constexpr int SUB_CHUNKS_P = SUB_BYTES_P / 16;
  constexpr int WIDEN = SUB_CHUNKS / SUB_CHUNKS_P;          // LDS chunks per pool chunk
  static_assert(WIDEN == 1 || (WIDEN == 2 && KV == PKV_FP8_E4M3FN), "staging widening");
  constexpr int NSB = BS / 16;
  constexpr int64_t REGION = int64_t(BS) * D * KvTraits<KV>::EB;   // in the pool
  constexpr int SUBS = step_subtiles<CKV, D>();
  constexpr int STEP_TOK = 16 * SUBS;
  constexpr int COLS = kWaves * 16 * CT;
  constexpr int STAGE_CHUNKS = 2 * SUBS * SUB_CHUNKS;       // K then V, in LDS
  constexpr int FETCH_CHUNKS = 2 * SUBS * SUB_CHUNKS_P;     // K then V, from the pool
  constexpr int PER_THREAD = FETCH_CHUNKS / kThreads;
  static_assert(FETCH_CHUNKS % kThreads == 0, "staging tiling");
  __shared__ __attribute__((aligned(16))) uint4 stage[2][STAGE_CHUNKS];
  extern __shared__ int32_t s_tbl[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup b runs on XCD b % kXcds, as its slot b / kXcds there.  With a plan, the
  // slots of an XCD hold its tiles longest first (the plan pass below); otherwise they follow
  // the default order of tile_job.  Either way a tile's output is the same.
  const int xcd = int(blockIdx.x) % kXcds, j = int(blockIdx.x) / kXcds;
  const TileJob job = a.plan ? a.plan[int64_t(xcd) * a.per_xcd + j] : tile_job(a, xcd, j);
  if (job.unit < 0) return;
  const int s = job.unit / a.Hkv, g = job.unit % a.Hkv;
  const int tile = job.tile, q0 = job.q0, n = job.n, L = job.L;
  const int col0 = tile * COLS;
  const int last_q = std::min(n - 1, (col0 + COLS - 1) / a.G);
  const int ntok = std::max(L - n + last_q + 1, 0);      // keys the workgroup reads
  const int nsub = (ntok + 15) / 16;
  const int nsteps = (nsub + SUBS - 1) / SUBS;
  const int nblk = (ntok + BS - 1) / BS;

  // The table entries the workgroup reads, then kTblPad entries of -1: a step's lookups
  // past the last block land there instead of outside the array.
  const int32_t* trow = a.block_tables + int64_t(s) * a.max_blocks;
  // Entries are kept as phys * Hkv (the block's first kv-head region), or -1 for an entry
  // outside [0, num_blocks): a staged chunk's address is then one shift and add.
  for (int e = tid; e < nblk + kTblPad; e += kThreads) {
    const int phys = e < nblk ? trow[e] : -1;
    s_tbl[e] = unsigned(phys) < unsigned(a.num_blocks) ? phys * a.Hkv : -1;
  }

  // This lane's columns: (query qi, head hh) for column col0 + 16*(wave*CT + ct) + lane%16.
  const int row = lane >> 4;
  int pos[CT];
  int wave_pmax = -1;
  uint4 qf[CT][F::NLOAD * F::QCH];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int c = col0 + 16 * (wave * CT + ct) + (lane & 15);
    const int qi = c / a.G, hh = c % a.G;
    const bool ok = qi < n;
    // A column past the sequence's queries is computed unmasked (over q = 0, finite) and
    // never written; it does not extend the wave's key range.
    pos[ct] = ok ? L - n + qi : INT32_MAX;
    wave_pmax = std::max(wave_pmax, ok ? pos[ct] : -1);
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                          ((int64_t(q0) + qi) * a.Hkv * a.G + int64_t(g) * a.G + hh) * D * T::QB;
#pragma unroll
    for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
      for (int cc = 0; cc < F::QCH; ++cc)
        qf[ct][i * F::QCH + cc] =
            ok ? *reinterpret_cast<const uint4*>(qrow + (int64_t(X) * (4 * i + row)) * T::QB + 16 * cc)
               : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wave_pmax = std::max(wave_pmax, __shfl_xor(wave_pmax, o));
  wave_pmax = __builtin_amdgcn_readfirstlane(wave_pmax);

  // Running max in raw logit units (before the scale), sum and accumulators per column.
  f32x4 acc[CT][F::NT];
  float m_run[CT], l_run[CT];
  // Kept with m_run and changed only when it is: the exponent offset -m_run * sl2 (0 while
  // nothing was seen) and the rescale threshold m_run + 8 / sl2 (raw logit units).
  float m_off[CT], thr[CT];
  // bf16 caches: the running sum of each column comes from the matrix unit, as the product
  // of an all-ones A operand with the same bf16 probabilities PV uses; every row of lsum[ct]
  // then holds the sum of column lane % 16 (fp8 caches are staged as bf16, so they too).
  f32x4 lsum[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int nn = 0; nn < F::NT; ++nn) acc[ct][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
    m_off[ct] = 0.f;
    thr[ct] = -INFINITY;
    lsum[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr bool MSUM = CKV == PKV_BF16;
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  const uint8_t* kbase = a.k_cache + int64_t(g) * REGION;
  const uint8_t* vbase = a.v_cache + int64_t(g) * REGION;
  __syncthreads();   // s_tbl

  // Chunk tid + kThreads*r of a step: K or V, sub-tile u, chunk w.  Sub-tiles past the keys the
  // workgroup reads and blocks outside [0, num_blocks) are read from block 0 (always in
  // bounds) and staged as zeros; zmask marks them (rare: the last step, or a bad table entry).
  //
  // LDS layout of a step: K sub-tiles in pool order, then V.  For bf16 the V chunks of each
  // pair of sub-tiles (2p, 2p+1) are interleaved by 8-byte halves, [pair][half e][chunk w]
  // [sub-tile parity]: one 16-byte read of (p, e, w) is then exactly the k = 32 PV operand
  // {sub-tile 2p half e, sub-tile 2p+1 half e} of output tile 2i+e, with no register moves.
  constexpr bool VPAIR = CKV == PKV_BF16;
  __builtin_assume(tid < kThreads);
  uint4 pre[PER_THREAD];
  uint32_t zmask = 0;
  auto fetch = [&](int step) {
    zmask = 0;
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = tid + kThreads * r;
      const int which = ci / (SUBS * SUB_CHUNKS_P);
      const int u = (ci / SUB_CHUNKS_P) % SUBS;
      const int w = ci % SUB_CHUNKS_P;
      const int k = step * SUBS + u;
      // k / NSB < nblk + 7 (a step starts below nsub), inside the padded table.
      const int region = s_tbl[k / NSB];
      const bool ok = k < nsub && region >= 0;
      zmask |= ok ? 0u : 1u << r;
      pre[r] = *reinterpret_cast<const uint4*>(
          (which ? vbase : kbase) + (ok ? int64_t(uint32_t(region)) * REGION + (k % NSB) * SUB_BYTES_P : 0) +
          w * 16);
    }
  };
  auto stage_write = [&](uint4* buf) {
    if (__any(zmask != 0)) {
#pragma unroll
      for (int r = 0; r < PER_THREAD; ++r)
        if ((zmask >> r) & 1u) pre[r] = make_uint4(0u, 0u, 0u, 0u);
    }
    // LDS chunk w of sub-tile u of K (which 0) or V (which 1).
    auto put = [&](int which, int u, int w, uint4 val) {
      if (!VPAIR || which == 0) {
        buf[(which * SUBS + u) * SUB_CHUNKS + w] = val;
      } else {
        uint2* vb = reinterpret_cast<uint2*>(buf + SUBS * SUB_CHUNKS);
        const int base = (u >> 1) * 2 * SUB_CHUNKS;
        vb[2 * (base + w) + (u & 1)] = make_uint2(val.x, val.y);
        vb[2 * (base + SUB_CHUNKS + w) + (u & 1)] = make_uint2(val.z, val.w);
      }
    };
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = tid + kThreads * r;
      const int which = ci / (SUBS * SUB_CHUNKS_P);
      const int u = (ci / SUB_CHUNKS_P) % SUBS, w = ci % SUB_CHUNKS_P;
      if constexpr (WIDEN == 1) {
        put(which, u, w, pre[r]);
      } else {
        // An fp8 chunk (64i + l) widens to two bf16 chunks; lo holds its bytes 0..7, hi 8..15.
        const uint4 lo = make_uint4(fp8x2_to_bf16x2<false>(pre[r].x), fp8x2_to_bf16x2<true>(pre[r].x),
                                    fp8x2_to_bf16x2<false>(pre[r].y), fp8x2_to_bf16x2<true>(pre[r].y));
        const uint4 hi = make_uint4(fp8x2_to_bf16x2<false>(pre[r].z), fp8x2_to_bf16x2<true>(pre[r].z),
                                    fp8x2_to_bf16x2<false>(pre[r].w), fp8x2_to_bf16x2<true>(pre[r].w));
        const int i = w >> 6, l = w & 63;
        if (which == 0) {
          // K: token l % 16, dims 16 (4i + l/16) .. +16, i.e. bf16 dim groups q and q + 1 of
          // 8, which are LDS chunks 64 (q/4) + 16 (q%4) + l % 16.
          const int q = 2 * (4 * i + (l >> 4)), t = l & 15;
          put(0, u, 64 * (q >> 2) + 16 * (q & 3) + t, lo);
          put(0, u, 64 * ((q + 1) >> 2) + 16 * ((q + 1) & 3) + t, hi);
        } else {
          // V: dims 64i + 16e + l % 16 for e = 0..3 (tokens 4 (l/16) .. +3): e = 0, 1 are
          // bf16 chunk 64 (2i) + l, e = 2, 3 chunk 64 (2i + 1) + l.
          put(1, u, 64 * (2 * i) + l, lo);
          put(1, u, 64 * (2 * i + 1) + l, hi);
        }
      }
    }
  };

  // One step's work for this wave; MASK: apply the causal mask and zero V of slots at or
  // past L (the steps on the diagonal and the last ones).  The running softmax is updated
  // once per UPD sub-tiles (64 tokens): every QK product of the update is issued first, then
  // one branch decides on the (rare) rescale for all column tiles, and the exponentials and
  // PV products of the update's sub-tile pairs follow in one straight run, so the compiler
  // can overlap one pair's exponentials with the previous pair's matrix instructions.
  const float sl2 = a.qk_scale_log2;
  const float grow_raw = 8.f / sl2;   // 2^8 in probability, in raw logit units
  constexpr int UPD = SUBS < 4 ? SUBS : 4;
  static_assert(SUBS % UPD == 0 && UPD % 2 == 0, "softmax update tiling");
  auto compute = [&](const uint4* buf, int tok_step, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool TAIL = MASK;
#pragma unroll
    for (int ub = 0; ub < SUBS; ub += UPD) {
      float sc[CT][UPD][4];   // raw logits; -inf where masked
      // The two waves of a SIMD run in step (one barrier per step); a raised priority while a
      // wave issues its matrix instructions lets the other wave's vector work fill the gaps.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int uu = 0; uu < UPD; ++uu) {
        const int u = ub + uu;
        uint4 kf[F::NLOAD];
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i) kf[i] = buf[u * SUB_CHUNKS + 64 * i + lane];
        const int t0 = tok_step + 16 * u + 4 * row;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x4 c = qk_subtile<CKV, D>(kf, qf[ct]);
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[ct][uu][j] = !MASK || t0 + j <= pos[ct] ? c[j] : -INFINITY;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // Each lane first checks only its own scores: a column's max grew by more than 2^8 in
      // probability exactly when one of the lanes holding that column sees such a score, so
      // the wave-wide vote below takes the same decision as the column maxima would, and the
      // cross-row reduction is needed only in the (rare) rescale.
      float lmax[CT];
      bool grow = false;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float v = -INFINITY;
#pragma unroll
        for (int uu = 0; uu < UPD; ++uu)
#pragma unroll
          for (int j = 0; j < 4; ++j) v = fmaxf(v, sc[ct][uu][j]);
        lmax[ct] = v;
        grow |= v > thr[ct];
      }
      // The accumulators are rescaled only when some column's max grew by more than 2^8 in
      // probability: until then p = 2^(s - m) stays below 256, which float32 sums and bf16
      // operands hold without loss of relative precision.
      if (__any(grow)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float m_new = fmaxf(m_run[ct], wave_max_rows(lmax[ct]));
          const float alpha = m_new == m_run[ct] ? 1.f : __builtin_amdgcn_exp2f((m_run[ct] - m_new) * sl2);
          m_run[ct] = m_new;
          m_off[ct] = m_new == -INFINITY ? 0.f : -m_new * sl2;
          thr[ct] = m_new + grow_raw;
          if constexpr (MSUM) lsum[ct] *= alpha;
          else l_run[ct] *= alpha;
#pragma unroll
          for (int nn = 0; nn < F::NT; ++nn) acc[ct][nn] *= alpha;
        }
      }
#pragma unroll
      for (int u0 = ub; u0 < ub + UPD; u0 += 2) {
        const int pu = u0 - ub;
        float p[CT][2][4];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              p[ct][uu][j] = __builtin_amdgcn_exp2f(fmaf(sc[ct][pu + uu][j], sl2, m_off[ct]));   // 0 where masked
              if constexpr (!MSUM) l_run[ct] += p[ct][uu][j];
            }
        const uint4* vsrc = buf + SUBS * SUB_CHUNKS;
        if constexpr (VPAIR) {
          // vp[e][i]: the paired operand of output tile 2i+e.
          uint4 vp[2][F::NLOAD];
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < F::NLOAD; ++i) vp[e][i] = vsrc[(u0 + e) * SUB_CHUNKS + 64 * i + lane];
          if constexpr (TAIL) {
            // Element order within a paired operand: tokens 4r..4r+3 of the first sub-tile,
            // then of the second.
            const int t0 = tok_step + 16 * u0 + 4 * row;
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              lo |= (t0 + j < L ? 0xFFFFu : 0u) << (16 * j);
              hi |= (t0 + 2 + j < L ? 0xFFFFu : 0u) << (16 * j);
            }
            uint32_t lo1 = 0, hi1 = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              lo1 |= (t0 + 16 + j < L ? 0xFFFFu : 0u) << (16 * j);
              hi1 |= (t0 + 18 + j < L ? 0xFFFFu : 0u) << (16 * j);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int i = 0; i < F::NLOAD; ++i) {
                vp[e][i].x &= lo; vp[e][i].y &= hi; vp[e][i].z &= lo1; vp[e][i].w &= hi1;
              }
          }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const uint4 bop = make_uint4(pack_bf16x2(p[ct][0][0], p[ct][0][1]), pack_bf16x2(p[ct][0][2], p[ct][0][3]),
                                         pack_bf16x2(p[ct][1][0], p[ct][1][1]), pack_bf16x2(p[ct][1][2], p[ct][1][3]));
            lsum[ct] = mfma_bf16_k32(ones, bop, lsum[ct]);
#pragma unroll
            for (int i = 0; i < F::NLOAD; ++i) {
              acc[ct][2 * i + 0] = mfma_bf16_k32(vp[0][i], bop, acc[ct][2 * i + 0]);
              acc[ct][2 * i + 1] = mfma_bf16_k32(vp[1][i], bop, acc[ct][2 * i + 1]);
            }
          }
          __builtin_amdgcn_s_setprio(0);
        } else {
          uint4 vf0[F::NLOAD], vf1[F::NLOAD];
#pragma unroll
          for (int i = 0; i < F::NLOAD; ++i) {
            vf0[i] = vsrc[u0 * SUB_CHUNKS + 64 * i + lane];
            vf1[i] = vsrc[(u0 + 1) * SUB_CHUNKS + 64 * i + lane];
          }
          if constexpr (TAIL) {
            const int t0 = tok_step + 16 * u0 + 4 * row;
            uint32_t vm0 = 0, vm1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              vm0 |= (t0 + j < L ? 1u : 0u) << j;
              vm1 |= (t0 + 16 + j < L ? 1u : 0u) << j;
            }
            mask_v<CKV, D>(vf0, vm0);
            mask_v<CKV, D>(vf1, vm1);
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) pv_pair<CKV, D>(acc[ct], vf0, vf1, p[ct][0], p[ct][1]);
        }
      }
    }
  };

  // Steps [0, s_free) lie below every column's position in the workgroup and need no mask;
  // the rest (the diagonal and the tail) are masked.  Two loops keep the two variants'
  // registers apart.  Each step: stage the loaded chunks, issue the next step's loads,
  // barrier, compute.
  const int pmin_wg = L - n + col0 / a.G;
  const int s_free = pmin_wg < 0 ? 0 : std::min(nsteps, (pmin_wg + 1) / STEP_TOK);
  auto run_steps = [&](int s_begin, int s_end, auto mask_c) {
    for (int step = s_begin; step < s_end; ++step) {
      uint4* buf = stage[step & 1];
      stage_write(buf);
      if (step + 1 < nsteps) fetch(step + 1);
      __syncthreads();
      const int tok_step = step * STEP_TOK;
      if (tok_step <= wave_pmax) compute(buf, tok_step, mask_c);
    }
  };
  if (nsteps > 0) fetch(0);
  run_steps(0, s_free, std::integral_constant<bool, false>());
  run_steps(s_free, nsteps, std::integral_constant<bool, true>());

#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float l_tot = MSUM ? lsum[ct][0] : wave_sum_rows(l_run[ct]);
    const int c = col0 + 16 * (wave * CT + ct) + (lane & 15);
    const int qi = c / a.G, hh = c % a.G;
    if (qi >= n) continue;
    const float inv = l_tot > 0.f ? a.v_scale / l_tot : 0.f;
    const int64_t orow = ((int64_t(q0) + qi) * a.Hkv * a.G + int64_t(g) * a.G + hh) * D;
#pragma unroll
    for (int nn = 0; nn < F::NT; ++nn) {
      const int d = 16 * nn + 4 * row;
      if constexpr (KV == PKV_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d) =
            make_float4(acc[ct][nn][0] * inv, acc[ct][nn][1] * inv, acc[ct][nn][2] * inv, acc[ct][nn][3] * inv);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d) =
            make_uint2(pack_bf16x2(acc[ct][nn][0] * inv, acc[ct][nn][1] * inv),
                       pack_bf16x2(acc[ct][nn][2] * inv, acc[ct][nn][3] * inv));
      }
    }
  }
}

// ---- launch order of the query tiles ------------------------------------------------------
//
// A workgroup holds a CU for as long as its tile takes, and a tile's time grows with the keys
// it reads.  In the default order an XCD runs its units in index order, so a long unit dealt
// late leaves a few CUs busy after the rest have drained.  The plan pass orders each XCD's
// units by the steps of their longest tile, longest first (a counting sort over step counts),
// and gives each unit a run of consecutive slots holding its tiles, last (longest) tile
// first; the slots of tiles with no query column go last.  Sorting whole units rather than
// single tiles keeps the tiles that run together on one unit, whose K/V then stays in the
// XCD's L2: an order of single tiles by length ran more units at once and lost more in L2
// misses than it gained in balance on full prompts.  Units with equal step counts take the
// order in which their atomic increments land, which changes the launch order but not what
// any tile computes.

constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 2048;   // step counts, shifted right by `shift` to fit
constexpr int kPlanUnits = 2048;     // units per XCD the plan orders, at most
constexpr int kPlanPerThread = kPlanUnits / kPlanThreads;
static_assert(kPlanUnits % kPlanThreads == 0, "plan tiling");

// In-place exclusive prefix sum of v[0..n) by the whole workgroup; returns the total.
__device__ int plan_exclusive_scan(int* v, int n, int* wave_total) {
  const int tid = int(threadIdx.x), lane = tid & 63;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = std::min(n, tid * per), hi = std::min(n, lo + per);
  int mine = 0;
  for (int r = lo; r < hi; ++r) mine += v[r];
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_total[tid >> 6] = incl;
  __syncthreads();
  int run = incl - mine, total = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    if (w < (tid >> 6)) run += wave_total[w];
    total += wave_total[w];
  }
  for (int r = lo; r < hi; ++r) {
    const int c = v[r];
    v[r] = run;
    run += c;
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPlanThreads) void paged_attention_prefill_plan_kernel(PrefillArgs a, int shift) {
  // Bucket r holds the units whose longest tile has the r-th largest step count; bucket
  // kPlanBuckets the units with no live tile.
  __shared__ int cursor[kPlanBuckets + 1];
  __shared__ int wave_total[kPlanThreads / 64];
  __shared__ int u_tiles[kPlanUnits];   // by unit (i: unit xcd + kXcds i): live tiles
  __shared__ SeqSpan u_span[kPlanUnits];
  __shared__ int r_unit[kPlanUnits];    // by place in the order: the unit
  __shared__ int r_first[kPlanUnits];   // by place: the unit's live tiles, then its first slot
  const int xcd = int(blockIdx.x), tid = int(threadIdx.x);
  const int U = a.units_per_xcd;
  for (int i = tid; i <= kPlanBuckets; i += kPlanThreads) cursor[i] = 0;
  __syncthreads();
  int bucket[kPlanPerThread];
#pragma unroll
  for (int k = 0; k < kPlanPerThread; ++k) {
    const int i = tid + k * kPlanThreads, unit = xcd + kXcds * i;
    bucket[k] = kPlanBuckets;
    if (i >= U) continue;
    int nt = 0;
    SeqSpan sp{0, 0, 0};
    if (unit < a.B * a.Hkv) {
      sp = seq_span(a, unit / a.Hkv);
      nt = live_tiles(a, sp);
      if (nt > 0)
        bucket[k] = kPlanBuckets - 1 - std::min(make_job(a, unit, nt - 1, sp).steps >> shift, kPlanBuckets - 1);
    }
    u_tiles[i] = nt;
    u_span[i] = sp;
    atomicAdd(&cursor[bucket[k]], 1);
  }
  __syncthreads();
  plan_exclusive_scan(cursor, kPlanBuckets + 1, wave_total);
#pragma unroll
  for (int k = 0; k < kPlanPerThread; ++k) {
    const int i = tid + k * kPlanThreads;
    if (i >= U) continue;
    const int r = atomicAdd(&cursor[bucket[k]], 1);
    r_unit[r] = i;
    r_first[r] = u_tiles[i];
  }
  __syncthreads();
  const int live = plan_exclusive_scan(r_first, U, wave_total);

  // Slots [0, live) hold the live tiles unit by unit in order, each unit's last tile first;
  // [live, per_xcd) nothing.  Places with live tiles come first, with increasing first
  // slots, so slot j's place is the last one whose first slot is <= j.
  TileJob* out = a.plan + int64_t(xcd) * a.per_xcd;
  for (int j = tid; j < a.per_xcd; j += kPlanThreads) {
    TileJob t{-1, 0, 0, 0, 0, 0, 0, 0};
    if (j < live) {
      int lo = 0, hi = U;   // r_first[lo] <= j < r_first[hi] (r_first[U] read as live)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (r_first[mid] <= j) lo = mid;
        else hi = mid;
      }
      const int i = r_unit[lo];
      t = make_job(a, xcd + kXcds * i, u_tiles[i] - 1 - (j - r_first[lo]), u_span[i]);
    }
    out[j] = t;
  }
}

// ---- few query tokens per sequence: split over the keys ---------------------------------
//
// With n_s * G <= 32 columns per (sequence, kv head) -- checking a few drafted tokens, or
// short prefill chunks -- a query tile would leave most of a workgroup idle and put one
// workgroup on each long (sequence, kv head).  This path is decode's: the flattened
// (sequence, kv head, block) list is cut into equal shares, one per wavefront; each wave
// streams its blocks straight from the pool (no LDS) with two 16-column matrix tiles
// covering all of the unit's (query, head) columns, the causal mask per column, and leaves
// a finished result or a partial (max, sum, accumulator) per column; a merge pass folds the
// partials of units that span several shares.

constexpr int kMqWaves = 4;
constexpr int kMqCols = 32;   // columns per (sequence, kv head) this path takes
// Batches of up to kMqScanSeqs sequences: each workgroup of the few-query split pass scans
// its work list into LDS, kMqScanSeqs / (kMqWaves * 64) sequences per thread.
constexpr int kMqScanSeqs = 512;
constexpr int kMqScanPerThread = kMqScanSeqs / (kMqWaves * 64);

struct MqArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  float* ws_acc;  // [splits*2][kMqCols][D]
  float* ws_ml;   // [splits*2][kMqCols][2]  (max in log2 units, sum)
  int* ws_seq;    // [B+1]: Hkv * blocks of the sequences before s; [B] = total work W
  int B, Hkv, G, num_blocks, max_blocks, num_q_tokens, splits;
  // Waves that walk one share together, each on its own kv head of the same blocks (a power
  // of two dividing Hkv and kMqWaves): the work list is (sequence, head group, block).
  int coop;
  float qk_scale_log2;
  float v_scale;
  const int32_t* shared_prefix;   // [B] or null: leading blocks other sequences also read
};

__device__ __forceinline__ int mq_len(const MqArgs& a, int s, int bs) {
  int L = a.context_lens[s];
  L = L < 0 ? 0 : L;
  const int64_t cap = int64_t(a.max_blocks) * bs;
  return L > cap ? int(cap) : L;
}

__device__ __forceinline__ void mq_queries(const MqArgs& a, int s, int& q0, int& n) {
  int lo = a.query_start[s], hi = a.query_start[s + 1];
  lo = std::min(std::max(lo, 0), a.num_q_tokens);
  hi = std::min(std::max(hi, lo), a.num_q_tokens);
  q0 = lo;
  n = hi - lo;
}

// The work list is cut by estimated cost, as decode's: a unit (one sequence's blocks for one
// group of kv heads) weighs kMqUnitW for its q and table round trip and its epilogue, plus
// kMqBlockW per block, and a block belongs to the share holding its first weighted position.
constexpr int kMqBlockW = 8;
constexpr int kMqUnitW = 12;

__device__ __forceinline__ int mq_span(int nb) { return nb > 0 ? nb * kMqBlockW + kMqUnitW : 0; }

// Blocks [j0, j1) of a unit (first weighted position unit_off, nb blocks) whose first weighted
// positions lie in [lo, hi).
__device__ __forceinline__ void mq_blocks_in(int unit_off, int nb, int lo, int hi, int& j0, int& j1) {
  const int base = unit_off + kMqUnitW;
  j0 = lo <= base ? 0 : std::min(nb, (lo - base + kMqBlockW - 1) / kMqBlockW);
  j1 = hi <= base ? 0 : std::min(nb, (hi - base + kMqBlockW - 1) / kMqBlockW);
}

// Total work W = kv-head groups * sum_s mq_span(blocks(s)) (wave-uniform).
__device__ int mq_total(const MqArgs& a, int bs, int lane) {
  int acc = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int s = base + lane;
    acc += s < a.B ? mq_span((mq_len(a, s, bs) + bs - 1) / bs) : 0;
  }
  return wave_sum(acc) * (a.Hkv / a.coop);
}

// Sequence whose units contain work position x, and the weighted positions before it.
__device__ void mq_locate(const MqArgs& a, int bs, int lane, int x, int& s_out, int& off_out) {
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int s = b0 + lane;
    const int w = s < a.B ? mq_span((mq_len(a, s, bs) + bs - 1) / bs) * (a.Hkv / a.coop) : 0;
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

// Partial (accumulator, max, sum) of column c in piece `piece`; lane (column c % 16, row)
// holds dims 16*nn + 4*row .. +3 of each 16-dim tile nn.  With bf16 or fp8 caches the
// accumulator is stored as bf16 (the output's precision; the sums and maxima stay float32),
// which halves the partial traffic.
template <int KV, int D>
__device__ __forceinline__ void store_mq_partial(const MqArgs& a, int64_t piece, int c, int row,
                                                 const f32x4* acc, float2 ml) {
  if constexpr (KV == PKV_F32) {
    float* wacc = a.ws_acc + (piece * kMqCols + c) * D;
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn)
      *reinterpret_cast<float4*>(wacc + 16 * nn + 4 * row) = make_float4(acc[nn][0], acc[nn][1], acc[nn][2], acc[nn][3]);
  } else {
    uint16_t* wacc = reinterpret_cast<uint16_t*>(a.ws_acc) + (piece * kMqCols + c) * D;
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn)
      *reinterpret_cast<uint2*>(wacc + 16 * nn + 4 * row) =
          make_uint2(pack_bf16x2(acc[nn][0], acc[nn][1]), pack_bf16x2(acc[nn][2], acc[nn][3]));
  }
  if (row == 0) *reinterpret_cast<float2*>(a.ws_ml + (piece * kMqCols + c) * 2) = ml;
}

template <int KV, int D, int BS, bool MIX>
__global__ __launch_bounds__(256, 2) void paged_attention_mq_split_kernel(MqArgs a) {
  using F = Frag<KV, D>;
  using T = KvTraits<KV>;
  constexpr int X = 16 / T::EB;
  constexpr int SUB_BYTES = 16 * D * T::EB;
  constexpr int NSB = BS / 16;
  constexpr int64_t REGION = int64_t(BS) * D * T::EB;
  constexpr int CT = kMqCols / 16;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Each XCD (workgroup b runs on XCD b % kXcds) takes a contiguous eighth of the work list;
  // shares and pieces are numbered by the logical wave.
  const int nwg = int(gridDim.x), full = nwg - nwg % kXcds;
  const int b = int(blockIdx.x);
  const int lwg = b < full ? (b % kXcds) * (full / kXcds) + b / kXcds : b;
  const int wave = lwg * kMqWaves + wv;
  // The partial of a share's first segment waits in LDS until the share's loads are done: a
  // wave's loads and stores complete in issue order, so a store in the middle of the share
  // would hold up every load behind it.  Each lane reads back only what it wrote.
  __shared__ f32x4 s_hold[kMqWaves][CT * F::NT][64];
  __shared__ float2 s_hold_ml[kMqWaves][CT][64];
  int hold_cols = 0;   // valid columns of the partial held in LDS (0: none)
  auto flush_hold = [&]() {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + (lane & 15);
      if (c >= hold_cols) continue;
      f32x4 h[F::NT];
#pragma unroll
      for (int nn = 0; nn < F::NT; ++nn) h[nn] = s_hold[wv][ct * F::NT + nn][lane];
      store_mq_partial<KV, D>(a, int64_t(wave) * 2, c, lane >> 4, h, s_hold_ml[wv][ct][lane]);
    }
    hold_cols = 0;
  };

  // The work list, scanned by the workgroup when the batch fits: exclusive prefix sums of the
  // per-unit spans ([B] on: the total), the clamped lengths and the query ranges, in LDS; a
  // wave then finds its share's first unit there and reads later units' entries there.
  __shared__ int s_off[kMqScanSeqs + 1];
  __shared__ int s_len[kMqScanSeqs];
  __shared__ int s_q0[kMqScanSeqs];
  __shared__ int s_qn[kMqScanSeqs];
  __shared__ int s_wsum[kMqWaves];
  const int hgs = a.Hkv / a.coop;
  const bool lds_lists = a.B <= kMqScanSeqs;
  int W;
  if (lds_lists) {
    const int tid = threadIdx.x;
    int len[kMqScanPerThread], sp[kMqScanPerThread], sum = 0;
#pragma unroll
    for (int r = 0; r < kMqScanPerThread; ++r) {
      const int sq = tid * kMqScanPerThread + r, sc = std::min(sq, a.B - 1);
      const int L = mq_len(a, sc, BS);
      int q0, n;
      mq_queries(a, sc, q0, n);
      len[r] = sq < a.B ? L : 0;
      sp[r] = mq_span((len[r] + BS - 1) / BS);
      sum += sp[r];
      s_q0[sq] = q0;
      s_qn[sq] = n;
    }
    const int incl = wave_incl_scan(sum, lane);
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int base = incl - sum, total = 0;
#pragma unroll
    for (int w = 0; w < kMqWaves; ++w) {
      base += w < wv ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
#pragma unroll
    for (int r = 0; r < kMqScanPerThread; ++r) {
      const int sq = tid * kMqScanPerThread + r;
      s_off[sq] = base;
      s_len[sq] = len[r];
      base += sp[r];
    }
    if (tid == 0) s_off[kMqScanSeqs] = total;
    __syncthreads();
    W = total * hgs;
  } else {
    W = mq_total(a, BS, lane);
  }
  if (wave == 0) {
    if (lds_lists) {
      for (int sq = lane; sq <= a.B; sq += 64) a.ws_seq[sq] = s_off[sq] * hgs;
    } else {
      int base = 0;
      for (int b0 = 0; b0 < a.B; b0 += 64) {
        const int sq = b0 + lane;
        const int w = sq < a.B ? mq_span((mq_len(a, sq, BS) + BS - 1) / BS) * hgs : 0;
        const int incl = wave_incl_scan(w, lane);
        if (sq < a.B) a.ws_seq[sq] = base + incl - w;
        base += __builtin_amdgcn_readlane(incl, 63);
      }
      if (lane == 0) a.ws_seq[a.B] = base;
    }
  }
  if (W == 0) return;
  // Share of this wave's group of `coop` consecutive waves, walked side by side on kv heads
  // coop*hg + sub, so that together they read the adjacent head regions of each block.
  // Pieces stay numbered per wave (2 * wave + slot).
  const int share = wave / a.coop, sub = wave % a.coop;
  // No share is shorter than one block's weight, so every share lying inside a unit holds a
  // block of it (the merge takes a piece from each share between the unit's first block and
  // its last).
  const int nshare = std::min(a.splits / a.coop, W / kMqBlockW);
  if (share >= nshare) return;
  const int c_begin = __builtin_amdgcn_readfirstlane(int(share_begin(share, W, nshare)));
  const int c_end = __builtin_amdgcn_readfirstlane(int(share_begin(share + 1, W, nshare)));

  int s, seq_off;
  if (lds_lists) {
    s = __builtin_amdgcn_readfirstlane(lds_search(s_off, a.B, hgs, c_begin, lane));
    seq_off = s_off[s] * hgs;
  } else {
    mq_locate(a, BS, lane, c_begin, s, seq_off);
  }
  if (s >= a.B) return;
  int L = lds_lists ? s_len[s] : mq_len(a, s, BS);
  int nb = (L + BS - 1) / BS;
  int span = mq_span(nb);
  int hg = (c_begin - seq_off) / span;
  int g = hg * a.coop + sub;
  int unit_off = seq_off + hg * span;
  int pos = c_begin;
  const int row = lane >> 4;
  const float sl2 = a.qk_scale_log2;

  while (pos < c_end) {
    const int unit_end = unit_off + span;
    const int seg_end = std::min(c_end, unit_end);
    int j0, j1;                                                          // blocks [j0, j1)
    mq_blocks_in(unit_off, nb, c_begin, c_end, j0, j1);
    if (j1 > j0) {
      const bool full = j0 == 0 && j1 == nb;
      const int k0 = j0 * NSB;
      const int k1 = (std::min(j1 * BS, L) + 15) / 16;                    // sub-tiles [k0, k1)

      // Sub-tiles below ks lie in blocks shared with other sequences: cached loads.
      const int ks = MIX ? std::min(__builtin_amdgcn_readfirstlane(a.shared_prefix[s]), nb) * NSB : 0;
      int q0, n;
      if (lds_lists) {
        q0 = s_q0[s];
        n = s_qn[s];
      } else {
        mq_queries(a, s, q0, n);
      }
      // Column c = 16*ct + lane%16 is (query c / G, head c % G); query i sits at L - n + i.
      int posc[CT];
      uint4 qf[CT][F::NLOAD * F::QCH];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + (lane & 15);
        const int qi = c / a.G, hh = c % a.G;
        const bool ok = qi < n;
        posc[ct] = ok ? L - n + qi : -1;
        const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                              ((int64_t(q0) + qi) * a.Hkv * a.G + int64_t(g) * a.G + hh) * D * T::QB;
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i)
#pragma unroll
          for (int cc = 0; cc < F::QCH; ++cc)
            qf[ct][i * F::QCH + cc] =
                ok ? *reinterpret_cast<const uint4*>(qrow + (int64_t(X) * (4 * i + row)) * T::QB + 16 * cc)
                   : make_uint4(0u, 0u, 0u, 0u);
      }
      const int32_t* trow = a.block_tables + int64_t(s) * a.max_blocks;
      int tbase = k0 / NSB;
      int tbl = tbase + lane < nb ? trow[tbase + lane] : -1;
      f32x4 acc[CT][F::NT];
      float m_run[CT], l_run[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int nn = 0; nn < F::NT; ++nn) acc[ct][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[ct] = -INFINITY;
        l_run[ct] = 0.f;
      }
      const uint8_t* kbase = a.k_cache + int64_t(g) * REGION;
      const uint8_t* vbase = a.v_cache + int64_t(g) * REGION;
      const int64_t block_stride = int64_t(a.Hkv) * REGION;

      for (int k = k0; k < k1; ++k) {
        if (k / NSB >= tbase + 64) {
          tbase = k / NSB;
          tbl = tbase + lane < nb ? trow[tbase + lane] : -1;
        }
        // K and V of the sub-tile are loaded together, with no branch before their use: a
        // table entry outside [0, num_blocks) reads block 0 and its keys and values are
        // replaced by zeros.
        const int phys = __builtin_amdgcn_readlane(tbl, k / NSB - tbase);
        const bool bad = unsigned(phys) >= unsigned(a.num_blocks);
        const int64_t off = (bad ? 0 : int64_t(phys) * block_stride) + (k % NSB) * SUB_BYTES + lane * 16;
        uint4 kf[F::NLOAD], vf[F::NLOAD];
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i) kf[i] = load_kv(kbase + off + i * 1024, MIX && k < ks);
#pragma unroll
        for (int i = 0; i < F::NLOAD; ++i) vf[i] = load_kv(vbase + off + i * 1024, MIX && k < ks);
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
            sc[j] = t0 + j <= posc[ct] ? c[j] * sl2 : -INFINITY;   // posc < L: the tail is masked too
            cmax = fmaxf(cmax, sc[j]);
          }
          cmax = wave_max_rows(cmax);
          const float m_new = fmaxf(m_run[ct], cmax);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;      // column with nothing yet
          const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_use);
          m_run[ct] = m_new;
          l_run[ct] *= alpha;
#pragma unroll
          for (int nn = 0; nn < F::NT; ++nn) acc[ct][nn] *= alpha;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[ct][j] = __builtin_amdgcn_exp2f(sc[j] - m_use);          // 0 where masked
            l_run[ct] += p[ct][j];
          }
        }
        uint32_t vm = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) vm |= (t0 + j < L && !bad ? 1u : 0u) << j;
        mask_v<KV, D>(vf, vm);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) pv_subtile<KV, D>(acc[ct], vf, p[ct]);
      }

      // The share's first segment (it begins within this unit's weight) is slot 0; any other
      // unfinished segment is the share's last, slot 1.
      const int slot = c_begin >= unit_off ? 0 : 1;
      const int64_t piece = int64_t(wave) * 2 + slot;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float l_tot = wave_sum_rows(l_run[ct]);
        const int c = 16 * ct + (lane & 15);
        const int qi = c / a.G, hh = c % a.G;
        if (qi >= n) continue;
        if (full) {
          const float inv = l_tot > 0.f ? a.v_scale / l_tot : 0.f;
          const int64_t orow = ((int64_t(q0) + qi) * a.Hkv * a.G + int64_t(g) * a.G + hh) * D;
#pragma unroll
          for (int nn = 0; nn < F::NT; ++nn) {
            const int d = 16 * nn + 4 * row;
            if constexpr (KV == PKV_F32) {
              *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d) =
                  make_float4(acc[ct][nn][0] * inv, acc[ct][nn][1] * inv, acc[ct][nn][2] * inv, acc[ct][nn][3] * inv);
            } else {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d) =
                  make_uint2(pack_bf16x2(acc[ct][nn][0] * inv, acc[ct][nn][1] * inv),
                             pack_bf16x2(acc[ct][nn][2] * inv, acc[ct][nn][3] * inv));
            }
          }
        } else if (slot == 0) {
#pragma unroll
          for (int nn = 0; nn < F::NT; ++nn) s_hold[wv][ct * F::NT + nn][lane] = acc[ct][nn];
          s_hold_ml[wv][ct][lane] = make_float2(m_run[ct], l_tot);
        } else {
          store_mq_partial<KV, D>(a, piece, c, row, acc[ct], make_float2(m_run[ct], l_tot));
        }
      }
      if (slot == 0 && !full) hold_cols = n * a.G;
    }

    pos = seg_end;
    if (pos >= c_end) break;
    // Next unit: next kv head of this sequence, else the next non-empty sequence.
    unit_off = unit_end;
    if (++hg == a.Hkv / a.coop) {
      hg = 0;
      bool done;
      do {
        done = ++s >= a.B;
      } while (!done && (L = lds_lists ? s_len[s] : mq_len(a, s, BS)) == 0);
      if (done) break;
      nb = (L + BS - 1) / BS;
      span = mq_span(nb);
    }
    g = hg * a.coop + sub;
  }

  if (hold_cols > 0) flush_hold();
}

// One wave per (four columns, kv head, sequence), four waves per workgroup: merges the
// partials of a split unit's columns, or writes zeros for the queries of a sequence without
// keys.  Lanes 16*i .. 16*i+15 take column c0 + i, each with D/16 consecutive dims, so every
// piece costs a lane two 16-byte loads and its column's (max, sum); a batch of pieces is
// requested before any is folded.
constexpr int kMqMergeCols = 4;
constexpr int kMqMergeWaves = 4;

template <int KV, int D, int BS>
__global__ __launch_bounds__(64 * kMqMergeWaves) void paged_attention_mq_merge_kernel(MqArgs a) {
  constexpr int EPL = D / 16;  // dims per lane
  constexpr int BATCH = 8;     // pieces per round of loads: a unit rarely spans more shares
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = (blockIdx.x * kMqMergeWaves + wave) * kMqMergeCols, g = blockIdx.y, s = blockIdx.z;
  int q0, n;
  mq_queries(a, s, q0, n);
  const int ncols = std::min(kMqMergeCols, n * a.G - c0);   // valid columns of this wave
  if (ncols <= 0) return;
  const bool col_ok = (lane >> 4) < ncols;
  const int c = c0 + std::min(lane >> 4, ncols - 1);         // this lane's column
  const int d0 = (lane & 15) * EPL;
  const int before = a.ws_seq[s];
  const int span = (a.ws_seq[s + 1] - before) / (a.Hkv / a.coop);   // weighted positions per unit
  const int nb = span > kMqUnitW ? (span - kMqUnitW) / kMqBlockW : 0;
  const int W = a.ws_seq[a.B];
  auto write = [&](const float* v, float inv) {
    if (!col_ok) return;
    const int qi = c / a.G, hh = c % a.G;
    const int64_t o = ((int64_t(q0) + qi) * a.Hkv * a.G + int64_t(g) * a.G + hh) * D + d0;
    if constexpr (KV == PKV_F32) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o + e) =
            make_float4(v[e] * inv, v[e + 1] * inv, v[e + 2] * inv, v[e + 3] * inv);
    } else {
      uint32_t w[EPL / 2];
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) w[e] = pack_bf16x2(v[2 * e] * inv, v[2 * e + 1] * inv);
      if constexpr (EPL == 8)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + o) = make_uint4(w[0], w[1], w[2], w[3]);
      else
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = make_uint2(w[0], w[1]);
    }
  };
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  if (nb == 0) {
    write(num, 0.f);
    return;
  }
  const int C = a.coop, sub = g % C;
  const int nshare = std::min(a.splits / C, W / kMqBlockW);
  const int off = before + (g / C) * span;
  // The shares holding the unit's first and last blocks (a block goes to the share of its
  // first weighted position).
  const int64_t wf = share_of(off + kMqUnitW, W, nshare),
                wl = share_of(off + kMqUnitW + (nb - 1) * kMqBlockW, W, nshare);
  if (wf == wl) return;
  const int np = int(wl - wf + 1);
  // Share w's pieces of kv head g are those of its wave C*w + g%C.  The unit's piece in share
  // wf is that share's first segment (slot 0) only if the share begins within the unit's
  // weight; in every later share it is the first segment.
  const int64_t piece0 = (wf * C + sub) * 2 + (share_begin(wf, W, nshare) >= off ? 0 : 1);
  float M = -INFINITY, den = 0.f;
  for (int j0 = 0; j0 < np; j0 += BATCH) {
    float2 ml[BATCH];
    float4 x[BATCH][EPL / 4];
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const int j = std::min(j0 + t, np - 1);
      const int64_t pc = j == 0 ? piece0 : ((wf + j) * C + sub) * 2;
      const int64_t r = pc * kMqCols + c;
      ml[t] = *reinterpret_cast<const float2*>(a.ws_ml + r * 2);
      if constexpr (KV == PKV_F32) {
        const float4* px = reinterpret_cast<const float4*>(a.ws_acc + r * D + d0);
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) x[t][i] = px[i];
      } else {
        // EPL bf16 values, 2 per dword.
        const uint32_t* pb = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(a.ws_acc) + r * D + d0);
        uint32_t w[EPL / 2];
        if constexpr (EPL == 8) {
          const uint4 v = *reinterpret_cast<const uint4*>(pb);
          w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(pb);
          w[0] = v.x; w[1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i)
          x[t][i] = make_float4(__uint_as_float(w[2 * i] << 16), __uint_as_float(w[2 * i] & 0xFFFF0000u),
                                __uint_as_float(w[2 * i + 1] << 16), __uint_as_float(w[2 * i + 1] & 0xFFFF0000u));
      }
    }
    float mb = M;
#pragma unroll
    for (int t = 0; t < BATCH; ++t)
      if (j0 + t < np) mb = fmaxf(mb, ml[t].x);
    if (mb == -INFINITY) continue;                   // nothing attended yet
    const float alpha = __builtin_amdgcn_exp2f(M - mb);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] *= alpha;
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      const float w = j0 + t < np ? __builtin_amdgcn_exp2f(ml[t].x - mb) : 0.f;
      den += ml[t].y * w;
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        num[4 * i + 0] += x[t][i].x * w;
        num[4 * i + 1] += x[t][i].y * w;
        num[4 * i + 2] += x[t][i].z * w;
        num[4 * i + 3] += x[t][i].w * w;
      }
    }
    M = mb;
  }
  write(num, den > 0.f ? a.v_scale / den : 0.f);
}

using MqFn = void (*)(MqArgs);
struct MqPair {
  MqFn split[2];   // [mixed]: 0 streams all K/V non-temporally, 1 caches shared leading blocks
  MqFn merge;
};

template <int KV, int D, int BS>
MqPair mq_kernels() {
  return {{paged_attention_mq_split_kernel<KV, D, BS, false>, paged_attention_mq_split_kernel<KV, D, BS, true>},
          paged_attention_mq_merge_kernel<KV, D, BS>};
}

bool pick_mq(pkv_dtype kv, int D, int bs, MqPair* kp) {
#define PKV_MQ(KVT, DD, BB) \
  if (kv == KVT && D == DD && bs == BB) { *kp = mq_kernels<KVT, DD, BB>(); return true; }
  PKV_MQ(PKV_F32, 64, 16) PKV_MQ(PKV_F32, 64, 32) PKV_MQ(PKV_F32, 128, 16) PKV_MQ(PKV_F32, 128, 32)
  PKV_MQ(PKV_BF16, 64, 16) PKV_MQ(PKV_BF16, 64, 32) PKV_MQ(PKV_BF16, 128, 16) PKV_MQ(PKV_BF16, 128, 32)
  PKV_MQ(PKV_FP8_E4M3FN, 64, 16) PKV_MQ(PKV_FP8_E4M3FN, 64, 32)
  PKV_MQ(PKV_FP8_E4M3FN, 128, 16) PKV_MQ(PKV_FP8_E4M3FN, 128, 32)
#undef PKV_MQ
  return false;
}

size_t mq_round(size_t b) { return (b + 255) / 256 * 256; }
size_t mq_workspace_bytes(int splits, int B, int D) {
  return mq_round(size_t(splits) * 2 * kMqCols * D * sizeof(float)) +
         mq_round(size_t(splits) * 2 * kMqCols * 2 * sizeof(float)) + (size_t(B) + 1) * sizeof(int);
}

// Default share count of the few-query path: as decode's, 2 workgroups of 4 waves per CU
// (4 for fp8 caches), capped by what the device keeps resident of the split kernel.
pkv_status mq_default_splits(const MqPair& kp, pkv_dtype kv, int* splits) {
  // The device queries are made once per (device, kernel) and cached.
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, std::pair<int, int>> cache;   // -> (CUs, resident)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return pkv::fail(PKV_HIP_ERROR, "pkv_paged_attention_prefill: no current device");
  }
  // The streaming variant: the share count must not depend on the load policy.
  const auto key = std::make_pair(dev, reinterpret_cast<const void*>(kp.split[0]));
  std::pair<int, int> cu_res;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it == cache.end()) {
      int cus = 0, per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, key.second, kMqWaves * 64, 0) != hipSuccess) {
        (void)hipGetLastError();
        return pkv::fail(PKV_HIP_ERROR, "pkv_paged_attention_prefill: device query failed");
      }
      it = cache.emplace(key, std::make_pair(cus, per_cu)).first;
    }
    cu_res = it->second;
  }
  const int target = kv == PKV_FP8_E4M3FN ? 4 : 2;
  *splits = std::max(1, cu_res.first * std::min(target, std::max(cu_res.second, 1)) * kMqWaves);
  return PKV_OK;
}

using PrefillFn = void (*)(PrefillArgs);

template <int KV, int D, int BS>
constexpr int prefill_col_tiles() {
  return KV == PKV_F32 ? 1 : 2;
}

template <int KV, int D, int BS>
PrefillFn prefill_fn() {
  return paged_attention_prefill_kernel<KV, D, BS, prefill_col_tiles<KV, D, BS>()>;
}

template <int KV>
bool pick_prefill(int D, int bs, PrefillFn* fn, int* cols, int* step_tok) {
  constexpr int CKV = KV == PKV_FP8_E4M3FN ? PKV_BF16 : KV;
  const int ct = KV == PKV_F32 ? 1 : 2;
  *cols = kWaves * 16 * ct;
  *step_tok = 16 * (D == 64 ? step_subtiles<CKV, 64>() : step_subtiles<CKV, 128>());
  if (D == 64 && bs == 16) *fn = prefill_fn<KV, 64, 16>();
  else if (D == 64 && bs == 32) *fn = prefill_fn<KV, 64, 32>();
  else if (D == 128 && bs == 16) *fn = prefill_fn<KV, 128, 16>();
  else if (D == 128 && bs == 32) *fn = prefill_fn<KV, 128, 32>();
  else return false;
  return true;
}

bool pick_prefill_any(pkv_dtype kv, int D, int bs, PrefillFn* fn, int* cols, int* step_tok) {
  return kv == PKV_F32    ? pick_prefill<PKV_F32>(D, bs, fn, cols, step_tok)
         : kv == PKV_BF16 ? pick_prefill<PKV_BF16>(D, bs, fn, cols, step_tok)
                          : pick_prefill<PKV_FP8_E4M3FN>(D, bs, fn, cols, step_tok);
}

// The tile path's grid: kXcds * units_per_xcd * tiles workgroup slots.
bool tile_grid(int B, int Hkv, int G, int max_query_len, int cols, int64_t* tiles, int64_t* per_xcd) {
  *tiles = (int64_t(max_query_len) * G + cols - 1) / cols;
  *per_xcd = (int64_t(B) * Hkv + kXcds - 1) / kXcds * *tiles;
  return *tiles <= int64_t(INT32_MAX) && *per_xcd <= int64_t(INT32_MAX) / kXcds;
}

// The plan's bytes, one TileJob per slot; 0 when an XCD has more units than the plan orders
// (the tiles then run in the default order).
size_t plan_bytes(int B, int Hkv, int64_t per_xcd) {
  if ((int64_t(B) * Hkv + kXcds - 1) / kXcds > kPlanUnits) return 0;
  return (size_t(kXcds) * per_xcd * sizeof(TileJob) + 255) / 256 * 256;
}

}  // namespace

namespace {

pkv_status check_mq_shape(const char* fn, int B, int num_q_tokens, int max_query_len, int Hq, int Hkv,
                          int head_dim, int block_size, pkv_dtype q_dtype, pkv_dtype kv_dtype) {
  if (B < 0 || num_q_tokens < 0 || max_query_len < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_seqs=%d num_q_tokens=%d max_query_len=%d Hq=%d Hkv=%d", fn,
                     B, num_q_tokens, max_query_len, Hq, Hkv);
  const bool combo_ok = (q_dtype == PKV_F32 && kv_dtype == PKV_F32) ||
                        (q_dtype == PKV_BF16 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3FN));
  if (!combo_ok)
    return pkv::fail(PKV_UNSUPPORTED, "%s: q_dtype=%d kv_dtype=%d", fn, int(q_dtype), int(kv_dtype));
  if (!((head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32)))
    return pkv::fail(PKV_UNSUPPORTED, "%s: head_dim=%d block_size=%d", fn, head_dim, block_size);
  return PKV_OK;
}

// The few-query path takes batches whose (query, head) columns per (sequence, kv head) fit
// two matrix tiles.
bool few_queries(int max_query_len, int G) { return int64_t(max_query_len) * G <= kMqCols; }

pkv_status mq_splits(const char* fn, pkv_dtype kv, int D, int bs, int requested, MqPair* kp, int* splits) {
  if (!pick_mq(kv, D, bs, kp)) return pkv::fail(PKV_UNSUPPORTED, "%s: no kernel for this shape", fn);
  if (requested < 0) return pkv::fail(PKV_INVALID_ARG, "%s: num_splits=%d", fn, requested);
  if (requested > 0) {
    *splits = requested;
    return PKV_OK;
  }
  return mq_default_splits(*kp, kv, splits);
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_prefill_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                                                 int head_dim, int block_size, pkv_dtype q_dtype,
                                                                 pkv_dtype kv_dtype, int max_query_len,
                                                                 int num_splits, size_t* bytes) {
  const char* fn = "pkv_paged_attention_prefill_workspace_size";
  if (!bytes) return pkv::fail(PKV_INVALID_ARG, "%s: null output", fn);
  pkv_status st = check_mq_shape(fn, num_seqs, 0, max_query_len, num_q_heads, num_kv_heads, head_dim,
                                 block_size, q_dtype, kv_dtype);
  if (st != PKV_OK) return st;
  *bytes = 0;
  if (!few_queries(max_query_len, num_q_heads / num_kv_heads)) {
    // The tile path's plan: optional, but the tiles then run longest first.
    PrefillFn kfn = nullptr;
    int cols = 0, step_tok = 0;
    int64_t tiles = 0, per_xcd = 0;
    if (!pick_prefill_any(kv_dtype, head_dim, block_size, &kfn, &cols, &step_tok))
      return pkv::fail(PKV_UNSUPPORTED, "%s: no kernel for this shape", fn);
    if (!tile_grid(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, max_query_len, cols, &tiles, &per_xcd))
      return pkv::fail(PKV_UNSUPPORTED, "%s: too many query tiles", fn);
    *bytes = plan_bytes(num_seqs, num_kv_heads, per_xcd);
    return PKV_OK;
  }
  MqPair kp;
  int splits = 0;
  if ((st = mq_splits(fn, kv_dtype, head_dim, block_size, num_splits, &kp, &splits)) != PKV_OK) return st;
  *bytes = mq_workspace_bytes(splits, num_seqs, head_dim);
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_attention_prefill(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* query_start, int num_seqs, int num_q_tokens,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    int max_blocks_per_seq, int max_query_len, float scale, float k_scale, float v_scale,
    pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits, void* workspace, size_t workspace_bytes,
    const int32_t* shared_prefix_blocks, void* stream) {
  const char* fn = "pkv_paged_attention_prefill";
  const int B = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads;
  pkv_status cst = check_mq_shape(fn, B, num_q_tokens, max_query_len, Hq, Hkv, head_dim, block_size, q_dtype,
                                  kv_dtype);
  if (cst != PKV_OK) return cst;
  if (num_blocks <= 0 || max_blocks_per_seq < 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_blocks=%d max_blocks_per_seq=%d", fn, num_blocks,
                     max_blocks_per_seq);
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f) || scale == INFINITY ||
      k_scale == INFINITY || v_scale == INFINITY)
    return pkv::fail(PKV_INVALID_ARG, "%s: scales must be positive and finite", fn);
  if (reinterpret_cast<uintptr_t>(shared_prefix_blocks) % 4 != 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: shared_prefix_blocks must be 4-byte aligned", fn);
  if (B == 0 || num_q_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || !query_start ||
      (max_blocks_per_seq > 0 && !block_tables))
    return pkv::fail(PKV_INVALID_ARG, "%s: null pointer", fn);
  if (!pkv::aligned16({out, q, k_cache, v_cache, workspace}))
    return pkv::fail(PKV_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (int64_t(B) * Hkv > int64_t(INT32_MAX))
    return pkv::fail(PKV_UNSUPPORTED, "%s: num_seqs * num_kv_heads exceeds 2^31", fn);
  if (int64_t(num_q_tokens) * Hq > int64_t(INT32_MAX) || int64_t(max_query_len) * (Hq / Hkv) > int64_t(INT32_MAX) / 2)
    return pkv::fail(PKV_UNSUPPORTED, "%s: too many query tokens", fn);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (few_queries(max_query_len, Hq / Hkv)) {
    // Few query tokens per sequence: shares of the (sequence, kv head, block) list, then merge.
    MqPair kp;
    int splits = 0;
    pkv_status st = mq_splits(fn, kv_dtype, head_dim, block_size, num_splits, &kp, &splits);
    if (st != PKV_OK) return st;
    const size_t need = mq_workspace_bytes(splits, B, head_dim);
    if (!workspace || workspace_bytes < need)
      return pkv::fail(PKV_INVALID_ARG, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
    if (B > 65535 || Hkv > 65535)
      return pkv::fail(PKV_UNSUPPORTED, "%s: num_seqs and num_kv_heads must be <= 65535 here", fn);
    if (int64_t(B) * Hkv * (int64_t(max_blocks_per_seq) * kMqBlockW + kMqUnitW) > int64_t(INT32_MAX))
      return pkv::fail(PKV_UNSUPPORTED,
                       "%s: num_seqs * max_blocks_per_seq * num_kv_heads is too large for the work list", fn);
    MqArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start = query_start;
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(wsb);
    a.ws_ml = reinterpret_cast<float*>(wsb + mq_round(size_t(splits) * 2 * kMqCols * head_dim * sizeof(float)));
    a.ws_seq = reinterpret_cast<int*>(wsb + mq_round(size_t(splits) * 2 * kMqCols * head_dim * sizeof(float)) +
                                      mq_round(size_t(splits) * 2 * kMqCols * 2 * sizeof(float)));
    a.B = B;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.num_q_tokens = num_q_tokens;
    a.splits = int(std::max<int64_t>(1, std::min<int64_t>(splits, int64_t(B) * Hkv * std::max(1, max_blocks_per_seq))));
    a.coop = 1;
    while (a.coop < kMqWaves && Hkv % (2 * a.coop) == 0 && a.splits >= 2 * a.coop) a.coop *= 2;
    a.qk_scale_log2 = scale * k_scale * kLog2e;
    a.v_scale = v_scale;
    a.shared_prefix = shared_prefix_blocks;
    const int mixed = shared_prefix_blocks != nullptr ? 1 : 0;
    const unsigned wgs = unsigned((int64_t(a.splits) + kMqWaves - 1) / kMqWaves);
    void *ev0 = nullptr, *ev1 = nullptr;
    if (pkv::take_launch_events(&ev0, &ev1)) {
      void* kargs[] = {&a};
      hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kp.split[mixed]), dim3(wgs),
                                        dim3(kMqWaves * 64),
                                        kargs, 0, hs, static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0);
      if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: %s", fn, hipGetErrorString(e));
    } else {
      hipLaunchKernelGGL(kp.split[mixed], dim3(wgs), dim3(kMqWaves * 64), 0, hs, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: split launch: %s", fn, hipGetErrorString(e));
    static_assert(kMqCols % (kMqMergeCols * kMqMergeWaves) == 0, "merge tiling");
    hipLaunchKernelGGL(kp.merge, dim3(unsigned(kMqCols / (kMqMergeCols * kMqMergeWaves)), unsigned(Hkv), unsigned(B)),
                       dim3(64 * kMqMergeWaves), 0, hs, a);
    e = hipGetLastError();
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: merge launch: %s", fn, hipGetErrorString(e));
    return PKV_OK;
  }
  const int64_t tbl_bytes = (int64_t(max_blocks_per_seq) + kTblPad) * 4;
  if (int64_t(num_blocks) * Hkv > int64_t(INT32_MAX))
    return pkv::fail(PKV_UNSUPPORTED, "%s: num_blocks * num_kv_heads exceeds 2^31", fn);
  if (tbl_bytes > kMaxTableBytes)
    return pkv::fail(PKV_UNSUPPORTED, "%s: max_blocks_per_seq=%d exceeds %d", fn, max_blocks_per_seq,
                     kMaxTableBytes / 4 - kTblPad);

  PrefillFn kfn = nullptr;
  int cols = 0, step_tok = 0;
  if (!pick_prefill_any(kv_dtype, head_dim, block_size, &kfn, &cols, &step_tok))
    return pkv::fail(PKV_UNSUPPORTED, "%s: no kernel for this shape", fn);
  const int G = Hq / Hkv;
  int64_t tiles = 0, per_xcd = 0;
  if (!tile_grid(B, Hkv, G, max_query_len, cols, &tiles, &per_xcd))
    return pkv::fail(PKV_UNSUPPORTED, "%s: too many query tiles", fn);
  const size_t need = plan_bytes(B, Hkv, per_xcd);
  if (workspace && workspace_bytes < need)
    return pkv::fail(PKV_INVALID_ARG, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);

  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.B = B;
  a.Hkv = Hkv;
  a.G = G;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_tokens = num_q_tokens;
  a.qk_scale_log2 = scale * k_scale * kLog2e;
  a.v_scale = v_scale;
  a.tiles = int(tiles);
  a.units_per_xcd = (B * Hkv + kXcds - 1) / kXcds;
  a.per_xcd = int(per_xcd);
  a.cols = cols;
  a.step_tok = step_tok;
  a.max_tok = int64_t(max_blocks_per_seq) * block_size;
  a.plan = need > 0 ? static_cast<TileJob*>(workspace) : nullptr;
  const int64_t wgs = int64_t(kXcds) * per_xcd;
  const dim3 grid{unsigned(wgs)}, block{unsigned(kThreads)};
  if (a.plan) {
    // Step counts are bucketed exactly while the longest possible tile has fewer steps than
    // there are buckets, and coarsened by powers of two beyond.
    const int64_t max_steps = (a.max_tok + step_tok - 1) / step_tok;
    int shift = 0;
    while ((max_steps >> shift) >= kPlanBuckets) ++shift;
    hipLaunchKernelGGL(paged_attention_prefill_plan_kernel, dim3(kXcds), dim3(kPlanThreads), 0, hs, a, shift);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: plan launch: %s", fn, hipGetErrorString(e));
  }
  const size_t lds = size_t(tbl_bytes);
  void *ev0 = nullptr, *ev1 = nullptr;
  if (pkv::take_launch_events(&ev0, &ev1)) {
    // The dispatch itself records the events, so they time the kernel alone.
    void* kargs[] = {&a};
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kfn), grid, block, kargs, lds, hs,
                                      static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0);
    if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: %s", fn, hipGetErrorString(e));
  } else {
    hipLaunchKernelGGL(kfn, grid, block, lds, hs, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: %s", fn, hipGetErrorString(e));
  return PKV_OK;
}
