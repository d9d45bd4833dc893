// KV-cache write (slot-mapping scatter, optional fp8 e4m3fn quantisation) and the
// whole-block copy behind copy-on-write, for gfx950.
//
//  * "What is PagedAttention?" (qubittool glossary), "How It Works: Map Logical to
//    Physical Blocks": decode appends a token into the sequence's partly filled last
//    block, so a step writes one slot per sequence; a prefill writes many.
//  * "PagedAttention: Optimizing KV Cache in vLLM" (grasp.study), §4 "Advanced Benefit:
//    Zero-Cost Sharing with Copy-on-Write": the writer receives a fresh block holding the
//    shared block's contents, before its write proceeds.
//
// Pool layout (see include/pagedkv.h): per (block, kv head) a region of bs*D elements in
// 16-token sub-tiles; within a sub-tile K element (t, d) sits at ((d/x)*16 + t)*x + d%x
// and V element (t, d) at (((d/(4x))*4 + t/4)*16 + d%16)*x + ((d/16)%(x/4))*4 + t%4,
// with x = 16 / element bytes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv_codec.h"
#include "status.h"

namespace {

using pkv::e4m3fn_from_f32;

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) {
  return __uint_as_float(uint32_t(*p) << 16);
}

// Writes dims d0 .. d0+X of token n, kv head h, into slot `slot` (one thread's share of the
// per-token path).  K: the dims are one 16-byte chunk of the token's sub-tile; V: the X
// elements land in X chunks that are 16 bytes apart (same position inside each).
template <int EB, typename InT, bool QUANT>
__device__ __forceinline__ void write_token_group(const InT* __restrict__ k_new, const InT* __restrict__ v_new,
                                                  uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                  int64_t n, int h, int grp, int64_t slot, int Hkv, int D,
                                                  int bs, float k_inv, float v_inv) {
  constexpr int X = 16 / EB;
  const int64_t blk = slot / bs;
  const int off = int(slot % bs);
  const int u = off >> 4, t = off & 15;
  const int d0 = grp * X;
  const int64_t sub = ((blk * Hkv + h) * int64_t(bs) + int64_t(u) * 16) * D;  // element index
  const int64_t src = (n * Hkv + h) * D + d0;
  const int64_t kel = sub + (int64_t(grp) * 16 + t) * X;
  // V element (t, d0 + e) for e < X: all share i = d0/(4X) and position group (d0/16)%(X/4).
  const int vi = d0 / (4 * X), ve = (d0 / 16) % (X / 4), vc0 = d0 % 16;
  const int64_t vel0 = sub + ((int64_t(vi) * 4 + (t >> 2)) * 16 + vc0) * X + ve * 4 + (t & 3);
  if constexpr (!QUANT) {
    // Bit copies: EB == sizeof(InT).
    *reinterpret_cast<uint4*>(k_cache + kel * EB) = *reinterpret_cast<const uint4*>(k_new + src);
    const InT* vs = v_new + src;
    InT* vd = reinterpret_cast<InT*>(v_cache) + vel0;
#pragma unroll
    for (int e = 0; e < X; ++e) vd[int64_t(e) * X] = vs[e];
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < X; ++e)
      w[e >> 2] |= e4m3fn_from_f32(load_as_f32(k_new + src + e) * k_inv) << (8 * (e & 3));
    *reinterpret_cast<uint4*>(k_cache + kel) = make_uint4(w[0], w[1], w[2], w[3]);
    uint8_t* vd = v_cache + vel0;
#pragma unroll
    for (int e = 0; e < X; ++e)
      vd[int64_t(e) * X] = uint8_t(e4m3fn_from_f32(load_as_f32(v_new + src + e) * v_inv));
  }
}

template <typename InT, bool QUANT>
__device__ __forceinline__ uint32_t cache_element(InT x, float inv) {
  if constexpr (QUANT) return e4m3fn_from_f32(load_as_f32(&x) * inv);
  else if constexpr (sizeof(InT) == 4) return __float_as_uint(x);
  else return uint32_t(x);
}

// One workgroup per (16 consecutive tokens, kv head).  When the 16 tokens go to the 16 slots
// of one sub-tile in order (a prefill, or any run of appends that fills a sub-tile), the
// workgroup writes that sub-tile's K and V regions whole: every thread stores complete
// 16-byte chunks (K from one token's row, V assembled from the token rows staged in LDS),
// so the stores are contiguous instead of scattered 2-byte writes.  Any other slot pattern
// (decode appends, skipped or out-of-range slots, runs that cross sub-tiles) takes the
// per-token path.
template <int EB, typename InT, bool QUANT>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const InT* __restrict__ k_new, const InT* __restrict__ v_new, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int T, int Hkv, int D,
    int bs, int64_t num_slots, float k_inv, float v_inv) {
  constexpr int X = 16 / EB;
  __shared__ int64_t s_slot[16];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[16 * 128 * sizeof(InT)];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.x) * 16;
  const int cnt = int(T - n0 < 16 ? T - n0 : 16);
  if (tid < 16) s_slot[tid] = tid < cnt ? slots[n0 + tid] : -1;
  __syncthreads();
  const int64_t s0 = s_slot[0];
  bool whole = cnt == 16 && s0 >= 0 && s0 % 16 == 0 && s0 + 15 < num_slots;
#pragma unroll
  for (int i = 1; i < 16; ++i) whole = whole && s_slot[i] == s0 + i;

  if (whole) {
    const int64_t blk = s0 / bs;
    const int64_t sub = ((blk * Hkv + h) * int64_t(bs) + (s0 % bs)) * D;   // element index
    // Stage the 16 tokens' V rows (row-major [16][D] of InT) in LDS.
    const int row_chunks = D * int(sizeof(InT)) / 16;
    for (int c = tid; c < 16 * row_chunks; c += 256) {
      const int t = c / row_chunks, w = c % row_chunks;
      reinterpret_cast<uint4*>(s_v)[c] =
          reinterpret_cast<const uint4*>(v_new + ((n0 + t) * Hkv + h) * D)[w];
    }
    __syncthreads();
    const InT* sv = reinterpret_cast<const InT*>(s_v);
    for (int c = tid; c < D * EB; c += 256) {          // 16-byte chunks of the sub-tile
      // K chunk c: token c % 16, dims X*(c/16) .. +X.
      const int t = c & 15, d0 = X * (c >> 4);
      const InT* ks = k_new + ((n0 + t) * Hkv + h) * D + d0;
      uint4 kc;
      if constexpr (!QUANT) {
        kc = *reinterpret_cast<const uint4*>(ks);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < X; ++e) w[e >> 2] |= e4m3fn_from_f32(load_as_f32(ks + e) * k_inv) << (8 * (e & 3));
        kc = make_uint4(w[0], w[1], w[2], w[3]);
      }
      *reinterpret_cast<uint4*>(k_cache + (sub + int64_t(c) * X) * EB) = kc;
      // V chunk c: tokens 4*((c/16)%4) + j (j < 4), dims (c/64)*4X + 16e + c%16 (e < X/4);
      // element e*4 + j.
      const int tg = ((c >> 4) & 3) * 4, vd0 = (c >> 6) * 4 * X + (c & 15);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < X / 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = e * 4 + j;   // element index within the chunk
          const uint32_t bits = cache_element<InT, QUANT>(sv[(tg + j) * D + vd0 + 16 * e], v_inv);
          w[(p * EB) >> 2] |= (EB == 4 ? bits : bits & ((1u << (8 * EB)) - 1u)) << (8 * ((p * EB) & 3));
        }
      *reinterpret_cast<uint4*>(v_cache + (sub + int64_t(c) * X) * EB) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return;
  }
  const int groups = D / X;
  for (int idx = tid; idx < cnt * groups; idx += 256) {
    const int t = idx / groups, grp = idx % groups;
    const int64_t slot = s_slot[t];
    if (slot < 0 || slot >= num_slots) continue;
    write_token_group<EB, InT, QUANT>(k_new, v_new, k_cache, v_cache, n0 + t, h, grp, slot, Hkv, D, bs,
                                      k_inv, v_inv);
  }
}

// grid.y = pair; each workgroup copies a strided share of the K and V block regions.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t chunks_per_block) {
  const int32_t src = pairs[2 * blockIdx.y + 0];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t s0 = int64_t(src) * chunks_per_block, d0 = int64_t(dst) * chunks_per_block;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks_per_block;
       i += int64_t(gridDim.x) * blockDim.x) {
    k_cache[d0 + i] = k_cache[s0 + i];
    v_cache[d0 + i] = v_cache[s0 + i];
  }
}


// One thread per sequence: the device-side mirror of a decode step's allocator update.  The
// step gave sequence s one token at position lens[s] in slot slots[s]; that position's block
// table entry becomes the slot's block (a new block, a copy-on-write copy, or the same tail
// block again) and the length grows by one.  A negative slot means no token for s.
__global__ __launch_bounds__(256) void apply_append_kernel(int32_t* __restrict__ tables,
                                                           int32_t* __restrict__ lens,
                                                           const int64_t* __restrict__ slots, int n,
                                                           int max_blocks, int bs, int64_t num_slots) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const int64_t slot = slots[s];
  if (slot < 0 || slot >= num_slots) return;
  const int pos = lens[s];
  if (pos < 0 || pos / bs >= max_blocks || pos % bs != int(slot % bs)) return;
  tables[int64_t(s) * max_blocks + pos / bs] = int32_t(slot / bs);
  lens[s] = pos + 1;
}

int elem_bytes(pkv_dtype t) { return t == PKV_F32 ? 4 : t == PKV_BF16 ? 2 : t == PKV_FP8_E4M3FN ? 1 : 0; }

bool shape_ok(int D, int bs, pkv_dtype kv) {
  const int eb = elem_bytes(kv);
  if (!eb) return false;
  const int x = 16 / eb;
  return (D == 64 || D == 128) && (bs == 16 || bs == 32) && D % (4 * x) == 0;
}

pkv_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                         int num_kv_heads, int head_dim, int block_size,
                                         int num_blocks, pkv_dtype in_dtype, pkv_dtype kv_dtype,
                                         float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_INVALID_ARG, "pkv_kv_cache_write: num_tokens=%d num_kv_heads=%d num_blocks=%d",
                     num_tokens, num_kv_heads, num_blocks);
  if (!shape_ok(head_dim, block_size, kv_dtype))
    return pkv::fail(PKV_UNSUPPORTED, "pkv_kv_cache_write: head_dim=%d block_size=%d kv_dtype=%d",
                     head_dim, block_size, int(kv_dtype));
  const bool quant = kv_dtype == PKV_FP8_E4M3FN;
  if (quant ? !(in_dtype == PKV_F32 || in_dtype == PKV_BF16) : in_dtype != kv_dtype)
    return pkv::fail(PKV_UNSUPPORTED, "pkv_kv_cache_write: in_dtype=%d -> kv_dtype=%d",
                     int(in_dtype), int(kv_dtype));
  if (quant && !(k_scale > 0.0f && v_scale > 0.0f && k_scale < INFINITY && v_scale < INFINITY))
    return pkv::fail(PKV_INVALID_ARG, "pkv_kv_cache_write: fp8 scales must be positive and finite");
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return pkv::fail(PKV_INVALID_ARG, "pkv_kv_cache_write: null pointer");
  if (num_kv_heads > 65535) return pkv::fail(PKV_UNSUPPORTED, "pkv_kv_cache_write: num_kv_heads > 65535");
  const int64_t nwg = (int64_t(num_tokens) + 15) / 16;
  const int64_t num_slots = int64_t(num_blocks) * block_size;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const dim3 grid{unsigned(nwg), unsigned(num_kv_heads)}, block{256u};
  if (kv_dtype == PKV_F32) {
    hipLaunchKernelGGL((kv_cache_write_kernel<4, float, false>), grid, block, 0, st,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), kc, vc,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_slots,
                       1.0f, 1.0f);
  } else if (kv_dtype == PKV_BF16) {
    hipLaunchKernelGGL((kv_cache_write_kernel<2, uint16_t, false>), grid, block, 0, st,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       kc, vc, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                       num_slots, 1.0f, 1.0f);
  } else if (in_dtype == PKV_BF16) {
    hipLaunchKernelGGL((kv_cache_write_kernel<1, uint16_t, true>), grid, block, 0, st,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       kc, vc, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                       num_slots, k_inv, v_inv);
  } else {
    hipLaunchKernelGGL((kv_cache_write_kernel<1, float, true>), grid, block, 0, st,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), kc, vc,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_slots,
                       k_inv, v_inv);
  }
  return launch_status("pkv_kv_cache_write");
}

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                                      int num_pairs, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, pkv_dtype kv_dtype,
                                      void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_INVALID_ARG, "pkv_copy_blocks: num_pairs=%d num_kv_heads=%d num_blocks=%d",
                     num_pairs, num_kv_heads, num_blocks);
  if (!shape_ok(head_dim, block_size, kv_dtype))
    return pkv::fail(PKV_UNSUPPORTED, "pkv_copy_blocks: head_dim=%d block_size=%d kv_dtype=%d",
                     head_dim, block_size, int(kv_dtype));
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_mapping)
    return pkv::fail(PKV_INVALID_ARG, "pkv_copy_blocks: null pointer");
  if (num_pairs > 65535) return pkv::fail(PKV_INVALID_ARG, "pkv_copy_blocks: more than 65535 pairs");
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(kv_dtype);
  const int64_t chunks = block_bytes / 16;
  const int64_t per_wg = 256 * 4;
  const unsigned gx = unsigned(std::min<int64_t>((chunks + per_wg - 1) / per_wg, 1024));
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, unsigned(num_pairs)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), block_mapping, num_blocks, chunks);
  return launch_status("pkv_copy_blocks");
}

extern "C" pkv_status pkv_apply_append(int32_t* block_tables, int32_t* context_lens,
                                       const int64_t* slot_mapping, int num_seqs,
                                       int max_blocks_per_seq, int block_size, int num_blocks,
                                       void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_INVALID_ARG,
                     "pkv_apply_append: num_seqs=%d max_blocks_per_seq=%d block_size=%d num_blocks=%d",
                     num_seqs, max_blocks_per_seq, block_size, num_blocks);
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !slot_mapping)
    return pkv::fail(PKV_INVALID_ARG, "pkv_apply_append: null pointer");
  hipLaunchKernelGGL(apply_append_kernel, dim3(unsigned((num_seqs + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), block_tables, context_lens, slot_mapping,
                     num_seqs, max_blocks_per_seq, block_size, int64_t(num_blocks) * block_size);
  return launch_status("pkv_apply_append");
}
