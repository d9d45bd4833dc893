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

// The 16 fp8 codes of 16 consecutive input elements held in `raw` (sizeof(InT) 16-byte
// words, elements in memory order), packed into one 16-byte chunk.
template <typename InT>
__device__ __forceinline__ uint4 quantize16_regs(const uint4* raw, float inv) {
  constexpr int PER = 16 / int(sizeof(InT));   // elements per 16-byte word
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int l = 0; l < 16 / PER; ++l) {
    const uint32_t r[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = l * PER + i;
      float f;
      if constexpr (sizeof(InT) == 4) f = __uint_as_float(r[i]);
      else f = __uint_as_float((i & 1) ? (r[i >> 1] & 0xFFFF0000u) : (r[i >> 1] << 16));
      w[e >> 2] |= e4m3fn_from_f32(f * inv) << (8 * (e & 3));
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The same for 16 consecutive input elements at p (16-byte aligned).
template <typename InT>
__device__ __forceinline__ uint4 quantize16(const InT* p, float inv) {
  constexpr int WORDS = int(sizeof(InT));      // 16 elements = sizeof(InT) 16-byte words
  uint4 raw[WORDS];
#pragma unroll
  for (int l = 0; l < WORDS; ++l) raw[l] = reinterpret_cast<const uint4*>(p)[l];
  return quantize16_regs<InT>(raw, inv);
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
    *reinterpret_cast<uint4*>(k_cache + kel) = quantize16(k_new + src, k_inv);
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

// Threads per workgroup of the write kernel: one per 16-byte chunk of a sub-tile (D * b),
// kept within [64, 256].
constexpr int write_threads(int D, int EB) { return D * EB < 64 ? 64 : D * EB > 256 ? 256 : D * EB; }

// One workgroup per (16 consecutive tokens, kv head), the head varying fastest across
// workgroups so that neighbouring workgroups read neighbouring input rows and write
// neighbouring pool regions.  The workgroup owns tokens n0 .. n0+15.
//
// A run is 16 consecutive tokens whose slots are the 16 slots of one sub-tile in order (a
// prefill writes its sequences' full sub-tiles this way, and so does any run of appends that
// fills one).  Runs need not start at a multiple of 16 in the token list (sequences of a
// prefill have arbitrary lengths), and two runs never overlap (slots are distinct).  The
// workgroup that owns a run's first token writes the run's sub-tile whole: every thread
// stores complete 16-byte chunks (K from one token's row, V assembled from the token rows
// staged in LDS), so the stores are contiguous instead of scattered element writes.  Each
// workgroup therefore looks at the slots of tokens n0-15 .. n0+30: at most one run starts
// among its own tokens, and at most one run that started among the previous 15 tokens
// reaches into them.  Its own tokens that no run covers (decode appends, partial sub-tiles,
// skipped or out-of-range slots) take the per-token path.
template <int EB, typename InT, bool QUANT, int D>
__global__ __launch_bounds__(write_threads(D, EB)) void kv_cache_write_kernel(
    const InT* __restrict__ k_new, const InT* __restrict__ v_new, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int T, int Hkv, int bs,
    int64_t num_slots, float k_inv, float v_inv) {
  constexpr int X = 16 / EB;
  constexpr int NT = write_threads(D, EB);
  constexpr int ROW = D * int(sizeof(InT)) / 16;        // 16-byte words per token row
  __shared__ int64_t s_slot[48];                        // entry k: slot of token n0 - 16 + k
  __shared__ int s_run[2];
  __shared__ __attribute__((aligned(16))) uint4 s_v[16 * ROW];
  const int tid = threadIdx.x;
  const int h = int(blockIdx.x % unsigned(Hkv));
  const int64_t n0 = int64_t(blockIdx.x / unsigned(Hkv)) * 16;
  const int cnt = int(T - n0 < 16 ? T - n0 : 16);
  for (int k = tid; k < 48; k += NT) {
    const int64_t n = n0 - 16 + k;
    s_slot[k] = n >= 0 && n < T ? slots[n] : -1;
  }
  __syncthreads();
  if (tid < 64) {
    // Lane i < 31 tests whether a run starts at token n0 - 15 + i (entry i + 1).
    bool ok = false;
    if (tid < 31) {
      const int64_t s0 = s_slot[tid + 1];
      ok = s0 >= 0 && s0 % 16 == 0 && s0 + 15 < num_slots;
#pragma unroll
      for (int i = 1; i < 16; ++i) ok = ok && s_slot[tid + 1 + i] == s0 + i;
    }
    const uint64_t m = __ballot(ok);
    if (tid == 0) {
      const uint64_t own = (m >> 15) & 0xFFFFu;   // starts at n0 .. n0+15
      const uint64_t prev = m & 0x7FFFu;           // starts at n0-15 .. n0-1
      // Offset of the run starting among the own tokens, or -1.
      s_run[0] = own ? int(__builtin_ctzll(own)) : -1;
      // A run starting at n0-15+b covers own tokens 0 .. b.
      s_run[1] = prev ? 64 - int(__builtin_clzll(prev)) : 0;
    }
  }
  __syncthreads();
  const int r = s_run[0], covered = s_run[1];

  if (r >= 0) {
    const int64_t nr = n0 + r;                    // first token of the run
    const int64_t s0 = s_slot[r + 16];
    const int64_t blk = s0 / bs;
    const int64_t sub = ((blk * Hkv + h) * int64_t(bs) + (s0 % bs)) * D;   // element index
    // Stage the run's V rows (row-major [16][D] of InT) in LDS.
    for (int c = tid; c < 16 * ROW; c += NT)
      s_v[c] = reinterpret_cast<const uint4*>(v_new + ((nr + c / ROW) * Hkv + h) * D)[c % ROW];
    __syncthreads();
    const InT* sv = reinterpret_cast<const InT*>(s_v);
    for (int c = tid; c < D * EB; c += NT) {           // 16-byte chunks of the sub-tile
      // K chunk c: token c % 16, dims X*(c/16) .. +X.
      const int t = c & 15, d0 = X * (c >> 4);
      const InT* ks = k_new + ((nr + t) * Hkv + h) * D + d0;
      uint4 kc;
      if constexpr (!QUANT) kc = *reinterpret_cast<const uint4*>(ks);
      else kc = quantize16(ks, k_inv);
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
  }
  // Own tokens outside both runs: [covered, r) when a run starts here, else [covered, cnt).
  const int lo = covered, hi = r >= 0 ? r : cnt;
  constexpr int groups = D / X;
  for (int idx = lo * groups + tid; idx < hi * groups; idx += NT) {
    const int t = idx / groups, grp = idx % groups;
    const int64_t slot = s_slot[t + 16];
    if (slot < 0 || slot >= num_slots) continue;
    write_token_group<EB, InT, QUANT>(k_new, v_new, k_cache, v_cache, n0 + t, h, grp, slot, Hkv, D, bs,
                                      k_inv, v_inv);
  }
}

template <int EB, typename InT, bool QUANT>
void launch_write(int D, unsigned nwg, hipStream_t st, const void* k_new, const void* v_new,
                  uint8_t* kc, uint8_t* vc, const int64_t* slots, int T, int Hkv, int bs,
                  int64_t num_slots, float k_inv, float v_inv) {
  const auto* k = static_cast<const InT*>(k_new);
  const auto* v = static_cast<const InT*>(v_new);
  if (D == 64)
    hipLaunchKernelGGL((kv_cache_write_kernel<EB, InT, QUANT, 64>), dim3(nwg), dim3(write_threads(64, EB)),
                       0, st, k, v, kc, vc, slots, T, Hkv, bs, num_slots, k_inv, v_inv);
  else
    hipLaunchKernelGGL((kv_cache_write_kernel<EB, InT, QUANT, 128>), dim3(nwg), dim3(write_threads(128, EB)),
                       0, st, k, v, kc, vc, slots, T, Hkv, bs, num_slots, k_inv, v_inv);
}

// Whole-block copies from a source pool to a destination pool (the same pool for
// copy-on-write; a device pool and a pinned host pool for a swap).  grid.y strides over the
// pairs, grid.x over each block's 16-byte chunks.  A pair with an id outside its pool is
// skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* dst_k, uint4* dst_v, const uint4* src_k,
                                                          const uint4* src_v, const int32_t* __restrict__ pairs,
                                                          int num_pairs, int src_blocks, int dst_blocks,
                                                          int64_t chunks_per_block) {
  for (int p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int32_t src = pairs[2 * p + 0];
    const int32_t dst = pairs[2 * p + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
    const int64_t s0 = int64_t(src) * chunks_per_block, d0 = int64_t(dst) * chunks_per_block;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks_per_block;
         i += int64_t(gridDim.x) * blockDim.x) {
      const uint4 k = src_k[s0 + i];
      const uint4 v = src_v[s0 + i];
      dst_k[d0 + i] = k;
      dst_v[d0 + i] = v;
    }
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
  if (!pkv::aligned16({k_new, v_new, k_cache, v_cache}))
    return pkv::fail(PKV_INVALID_ARG, "pkv_kv_cache_write: tensor pointers must be 16-byte aligned");
  if ((int64_t(num_tokens) + 15) / 16 * num_kv_heads > int64_t(UINT32_MAX))
    return pkv::fail(PKV_UNSUPPORTED, "pkv_kv_cache_write: too many tokens x kv heads");
  const int64_t nwg = (int64_t(num_tokens) + 15) / 16;
  const int64_t num_slots = int64_t(num_blocks) * block_size;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const unsigned grid = unsigned(nwg * num_kv_heads);   // token groups x kv heads
  if (kv_dtype == PKV_F32)
    launch_write<4, float, false>(head_dim, grid, st, k_new, v_new, kc, vc, slot_mapping, num_tokens,
                                  num_kv_heads, block_size, num_slots, 1.0f, 1.0f);
  else if (kv_dtype == PKV_BF16)
    launch_write<2, uint16_t, false>(head_dim, grid, st, k_new, v_new, kc, vc, slot_mapping, num_tokens,
                                     num_kv_heads, block_size, num_slots, 1.0f, 1.0f);
  else if (in_dtype == PKV_BF16)
    launch_write<1, uint16_t, true>(head_dim, grid, st, k_new, v_new, kc, vc, slot_mapping, num_tokens,
                                    num_kv_heads, block_size, num_slots, k_inv, v_inv);
  else
    launch_write<1, float, true>(head_dim, grid, st, k_new, v_new, kc, vc, slot_mapping, num_tokens,
                                 num_kv_heads, block_size, num_slots, k_inv, v_inv);
  return launch_status("pkv_kv_cache_write");
}

namespace {

// Host-side checks shared by the block copies (nothing touches the device).
pkv_status check_copy(const char* fn, const void* dst_k, const void* dst_v, int dst_blocks, const void* src_k,
                      const void* src_v, int src_blocks, const int32_t* pairs, int num_pairs, int num_kv_heads,
                      int head_dim, int block_size, pkv_dtype kv_dtype) {
  if (num_pairs < 0 || num_kv_heads <= 0 || src_blocks <= 0 || dst_blocks <= 0)
    return pkv::fail(PKV_INVALID_ARG, "%s: num_pairs=%d num_kv_heads=%d pools of %d and %d blocks", fn,
                     num_pairs, num_kv_heads, src_blocks, dst_blocks);
  if (!shape_ok(head_dim, block_size, kv_dtype))
    return pkv::fail(PKV_UNSUPPORTED, "%s: head_dim=%d block_size=%d kv_dtype=%d", fn, head_dim,
                     block_size, int(kv_dtype));
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return pkv::fail(PKV_INVALID_ARG, "%s: null pointer", fn);
  if (!pkv::aligned16({dst_k, dst_v, src_k, src_v}))
    return pkv::fail(PKV_INVALID_ARG, "%s: pools must be 16-byte aligned", fn);
  return PKV_OK;
}

pkv_status launch_copy(const char* fn, void* dst_k, void* dst_v, int dst_blocks, const void* src_k,
                       const void* src_v, int src_blocks, const int32_t* pairs, int num_pairs,
                       int num_kv_heads, int head_dim, int block_size, pkv_dtype kv_dtype, void* stream) {
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(kv_dtype);
  const int64_t chunks = block_bytes / 16;
  const int64_t per_wg = 256 * 4;
  const unsigned gx = unsigned(std::min<int64_t>((chunks + per_wg - 1) / per_wg, 1024));
  const unsigned gy = unsigned(std::min(num_pairs, 65535));
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
                     static_cast<const uint4*>(src_v), pairs, num_pairs, src_blocks, dst_blocks, chunks);
  return launch_status(fn);
}

}  // namespace

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                                      int num_pairs, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, pkv_dtype kv_dtype,
                                      void* stream) {
  const char* fn = "pkv_copy_blocks";
  pkv_status st = check_copy(fn, k_cache, v_cache, num_blocks, k_cache, v_cache, num_blocks, block_mapping,
                             num_pairs, num_kv_heads, head_dim, block_size, kv_dtype);
  if (st != PKV_OK || num_pairs == 0) return st;
  return launch_copy(fn, k_cache, v_cache, num_blocks, k_cache, v_cache, num_blocks, block_mapping, num_pairs,
                     num_kv_heads, head_dim, block_size, kv_dtype, stream);
}

namespace {

// The address at which the device reaches `p`: device memory as it is, pinned host memory
// (hipHostMalloc) at the device address the runtime reports.  Anything else (pageable host
// memory, an unknown pointer) is rejected before any kernel could touch it.
pkv_status device_view(const char* fn, const char* name, const void* p, void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return pkv::fail(PKV_INVALID_ARG, "%s: %s is neither device memory nor pinned host memory", fn, name);
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(p);
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer && attr.hostPointer) {
    // Offset from the host address the runtime reports (the allocation's, or p itself).
    *out = static_cast<char*>(attr.devicePointer) +
           (static_cast<const char*>(p) - static_cast<const char*>(attr.hostPointer));
    return PKV_OK;
  }
  return pkv::fail(PKV_INVALID_ARG, "%s: %s is not device-accessible memory", fn, name);
}

}  // namespace

extern "C" pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int dst_num_blocks, const void* src_k,
                                      const void* src_v, int src_num_blocks, const int32_t* block_mapping,
                                      int num_pairs, int num_kv_heads, int head_dim, int block_size,
                                      pkv_dtype kv_dtype, void* stream) {
  const char* fn = "pkv_swap_blocks";
  pkv_status st = check_copy(fn, dst_k, dst_v, dst_num_blocks, src_k, src_v, src_num_blocks, block_mapping,
                             num_pairs, num_kv_heads, head_dim, block_size, kv_dtype);
  if (st != PKV_OK || num_pairs == 0) return st;
  void *dk, *dv, *sk, *sv, *map;
  if ((st = device_view(fn, "dst_k", dst_k, &dk)) != PKV_OK || (st = device_view(fn, "dst_v", dst_v, &dv)) != PKV_OK ||
      (st = device_view(fn, "src_k", src_k, &sk)) != PKV_OK || (st = device_view(fn, "src_v", src_v, &sv)) != PKV_OK ||
      (st = device_view(fn, "block_mapping", block_mapping, &map)) != PKV_OK)
    return st;
  return launch_copy(fn, dk, dv, dst_num_blocks, sk, sv, src_num_blocks, static_cast<const int32_t*>(map),
                     num_pairs, num_kv_heads, head_dim, block_size, kv_dtype, stream);
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
  // The slots may sit in pinned host memory: the kernel then reads them over the host link
  // (a few KiB), which saves the step a separate upload.
  void* slots = nullptr;
  pkv_status st = device_view("pkv_apply_append", "slot_mapping", slot_mapping, &slots);
  if (st != PKV_OK) return st;
  hipLaunchKernelGGL(apply_append_kernel, dim3(unsigned((num_seqs + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), block_tables, context_lens,
                     static_cast<const int64_t*>(slots), num_seqs, max_blocks_per_seq, block_size,
                     int64_t(num_blocks) * block_size);
  return launch_status("pkv_apply_append");
}
