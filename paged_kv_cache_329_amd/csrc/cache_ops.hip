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

// One thread per (token, kv head, group of x consecutive dims).  K: the group is one
// 16-byte chunk of the token's sub-tile; V: the group's x elements land in x chunks that
// are 16 bytes apart (same position inside each).
template <int EB, typename InT, bool QUANT>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const InT* __restrict__ k_new, const InT* __restrict__ v_new, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int T, int Hkv, int D,
    int bs, int64_t num_slots, float k_inv, float v_inv) {
  constexpr int X = 16 / EB;
  const int groups = D / X;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(T) * Hkv * groups;
  if (gid >= total) return;
  const int grp = int(gid % groups);
  const int h = int((gid / groups) % Hkv);
  const int64_t n = gid / (int64_t(groups) * Hkv);
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / bs;
  const int off = int(slot % bs);
  const int u = off >> 4, t = off & 15;
  const int d0 = grp * X;
  const int64_t region = (blk * Hkv + h) * int64_t(bs) * D;  // element index of the region
  const int64_t sub = region + int64_t(u) * 16 * D;
  const int64_t src = (n * Hkv + h) * D + d0;

  // K: one 16-byte chunk.
  const int64_t kel = sub + (int64_t(grp) * 16 + t) * X;
  // V: element (t, d0 + e) for e < X; all share i = d0/(4X), tile e4 = (d0/16)%(X/4).
  const int vi = d0 / (4 * X), ve = (d0 / 16) % (X / 4), vc0 = d0 % 16;
  const int64_t vel0 = sub + ((int64_t(vi) * 4 + (t >> 2)) * 16 + vc0) * X + ve * 4 + (t & 3);

  if constexpr (!QUANT) {
    // Bit copies: EB == sizeof(InT).
    const uint4 kv = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(k_cache + kel * EB) = kv;
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
  const int x = 16 / elem_bytes(kv_dtype);
  const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / x);
  const int64_t nwg = (total + 255) / 256;
  if (nwg > INT32_MAX) return pkv::fail(PKV_INVALID_ARG, "pkv_kv_cache_write: too many tokens");
  const int64_t num_slots = int64_t(num_blocks) * block_size;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const dim3 grid{unsigned(nwg)}, block{256u};
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
