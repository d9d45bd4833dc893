// Wavefront-level building blocks shared by the decode and the multi-query attention
// kernels: 16-token sub-tile operands of the pool layout fed to gfx950 matrix instructions.
//
// A 16-token sub-tile of one (block, kv head) is one contiguous region of 16 * D elements;
// wave load i, lane l reads its 16-byte chunk 64*i + l, which is exactly lane l's operand:
//   QK:  S^T[16 tokens][16 columns] = K[16 x D] . Q^T[D x 16]
//        A = K chunk (token l%16, dims of chunk 4i + l/16), B = the matching q dims of
//        column l%16;
//   PV:  O^T[16 dims][16 columns] += V^T[16 x 16 tokens] . P^T[16 tokens x 16 columns]
//        A = V chunk (4 tokens 4(l/16).. for dim l%16), B = the probabilities lane l holds
//        from QK (C layout: token 4(l/16)+j, column l%16).
// A column is one (query token, query head) pair; decode has one query token per column
// set, multi-query attention several.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pagedkv.h"

namespace pkv {
namespace tile {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

template <int KV>
struct KvTraits;
template <>
struct KvTraits<PKV_F32> {
  static constexpr int EB = 4;   // bytes per cached element
  static constexpr int QB = 4;   // bytes per q / out element
};
template <>
struct KvTraits<PKV_BF16> {
  static constexpr int EB = 2;
  static constexpr int QB = 2;
};
template <>
struct KvTraits<PKV_FP8_E4M3FN> {
  static constexpr int EB = 1;
  static constexpr int QB = 2;
};

// A 16-byte K/V chunk of a block read once per call: the load carries the non-temporal
// hint, which on MI355X lifts a random 4 KiB-chunk gather from about 5.9 to 6.5 TB/s,
// because streaming data no longer displaces cache lines.
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A chunk of a block that several sequences of the call read (a shared prefix): an ordinary
// cached load, so that the sequences reading it at about the same time can find it in L2 or
// the MALL.  `shared` is wave-uniform.
__device__ __forceinline__ uint4 load_kv(const uint8_t* p, bool shared) {
  return shared ? *reinterpret_cast<const uint4*>(p) : load_stream(p);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> two bf16 (round to nearest even) in one dword, lo in the low half
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two e4m3fn codes (bytes 2*sel, 2*sel+1 of w) -> two bf16 in one dword, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x4 mfma_bf16_k32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_k16(uint32_t a_lo, uint32_t a_hi, uint32_t b_lo,
                                               uint32_t b_hi, f32x4 c) {
  const uint2 a = make_uint2(a_lo, a_hi), b = make_uint2(b_lo, b_hi);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48 hold one
// column).  v_permlane16_swap exchanges the odd rows of one register with the even rows of
// the other and v_permlane32_swap the upper half of one with the lower half of the other, so
// applied to two copies of v they leave each lane holding v at l and at l^16 (then l^32).
__device__ __forceinline__ float wave_max_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the wave, returned as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Largest s in [0, n) with hg * e[s] <= x, for e non-decreasing in LDS with e[0] = 0: each
// step samples 64 evenly spaced entries of the remaining range.
__device__ __forceinline__ int lds_search(const int* e, int n, int hg, int x, int lane) {
  int lo = 0;
  while (n > 1) {
    const int step = (n + 63) / 64;
    const bool le = lane * step < n && hg * e[lo + lane * step] <= x;
    const int l = 63 - __builtin_clzll(__ballot(le));
    lo += l * step;
    n = std::min(step, n - l * step);
  }
  return lo;
}

// Equal shares of a work list of W positions cut into n: share w starts at w * W / n.
__device__ __forceinline__ int64_t share_begin(int64_t w, int64_t W, int64_t n) { return w * W / n; }

// Index of the share holding work position x.
__device__ __forceinline__ int64_t share_of(int64_t x, int64_t W, int64_t n) {
  return ((x + 1) * n - 1) / W;
}

template <int KV, int D>
struct Frag {
  using T = KvTraits<KV>;
  static constexpr int NLOAD = D * T::EB / 64;            // 16-byte chunks per lane per sub-tile
  static constexpr int QCH = (16 / T::EB) * T::QB / 16;   // 16-byte q chunks per K chunk
  static constexpr int NT = D / 16;                        // 16-dim output tiles
};

// S^T for one sub-tile: c[j] = <K[token 4(l/16)+j], Q[head l%16]>.
template <int KV, int D>
__device__ __forceinline__ f32x4 qk_subtile(const uint4* kf, const uint4* qf) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < Frag<KV, D>::NLOAD; ++i) {
    if constexpr (KV == PKV_F32) {
      c = mfma_f32_k4(__uint_as_float(kf[i].x), __uint_as_float(qf[i].x), c);
      c = mfma_f32_k4(__uint_as_float(kf[i].y), __uint_as_float(qf[i].y), c);
      c = mfma_f32_k4(__uint_as_float(kf[i].z), __uint_as_float(qf[i].z), c);
      c = mfma_f32_k4(__uint_as_float(kf[i].w), __uint_as_float(qf[i].w), c);
    } else if constexpr (KV == PKV_BF16) {
      c = mfma_bf16_k32(kf[i], qf[i], c);
    } else {
      const uint4 lo = make_uint4(fp8x2_to_bf16x2<false>(kf[i].x), fp8x2_to_bf16x2<true>(kf[i].x),
                                  fp8x2_to_bf16x2<false>(kf[i].y), fp8x2_to_bf16x2<true>(kf[i].y));
      const uint4 hi = make_uint4(fp8x2_to_bf16x2<false>(kf[i].z), fp8x2_to_bf16x2<true>(kf[i].z),
                                  fp8x2_to_bf16x2<false>(kf[i].w), fp8x2_to_bf16x2<true>(kf[i].w));
      c = mfma_bf16_k32(lo, qf[2 * i + 0], c);
      c = mfma_bf16_k32(hi, qf[2 * i + 1], c);
    }
  }
  return c;
}

// acc[n] += V^T tile n . P^T, p[j] = probability of token 4(l/16)+j for head l%16.
template <int KV, int D>
__device__ __forceinline__ void pv_subtile(f32x4* acc, const uint4* vf, const float* p) {
  if constexpr (KV == PKV_F32) {
#pragma unroll
    for (int i = 0; i < Frag<KV, D>::NLOAD; ++i) {
      acc[i] = mfma_f32_k4(__uint_as_float(vf[i].x), p[0], acc[i]);
      acc[i] = mfma_f32_k4(__uint_as_float(vf[i].y), p[1], acc[i]);
      acc[i] = mfma_f32_k4(__uint_as_float(vf[i].z), p[2], acc[i]);
      acc[i] = mfma_f32_k4(__uint_as_float(vf[i].w), p[3], acc[i]);
    }
  } else {
    const uint32_t b_lo = pack_bf16x2(p[0], p[1]), b_hi = pack_bf16x2(p[2], p[3]);
#pragma unroll
    for (int i = 0; i < Frag<KV, D>::NLOAD; ++i) {
      if constexpr (KV == PKV_BF16) {
        acc[2 * i + 0] = mfma_bf16_k16(vf[i].x, vf[i].y, b_lo, b_hi, acc[2 * i + 0]);
        acc[2 * i + 1] = mfma_bf16_k16(vf[i].z, vf[i].w, b_lo, b_hi, acc[2 * i + 1]);
      } else {
        const uint32_t w[4] = {vf[i].x, vf[i].y, vf[i].z, vf[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[4 * i + e] = mfma_bf16_k16(fp8x2_to_bf16x2<false>(w[e]), fp8x2_to_bf16x2<true>(w[e]),
                                         b_lo, b_hi, acc[4 * i + e]);
      }
    }
  }
}

// Zero the V elements of tokens 4(l/16)+j that are not valid (vmask bit j clear).
template <int KV, int D>
__device__ __forceinline__ void mask_v(uint4* vf, uint32_t vmask) {
  uint32_t m[4];
  if constexpr (KV == PKV_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = (vmask >> j) & 1u ? 0xFFFFFFFFu : 0u;
  } else if constexpr (KV == PKV_BF16) {
    const uint32_t m01 = ((vmask & 1u) ? 0x0000FFFFu : 0u) | ((vmask & 2u) ? 0xFFFF0000u : 0u);
    const uint32_t m23 = ((vmask & 4u) ? 0x0000FFFFu : 0u) | ((vmask & 8u) ? 0xFFFF0000u : 0u);
    m[0] = m01; m[1] = m23; m[2] = m01; m[3] = m23;
  } else {
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) b |= ((vmask >> j) & 1u) ? (0xFFu << (8 * j)) : 0u;
    m[0] = m[1] = m[2] = m[3] = b;
  }
#pragma unroll
  for (int i = 0; i < Frag<KV, D>::NLOAD; ++i) {
    vf[i].x &= m[0]; vf[i].y &= m[1]; vf[i].z &= m[2]; vf[i].w &= m[3];
  }
}


// acc[n] += V^T tile n . P^T over two sub-tiles at once (32 tokens, one k = 32 product per
// tile for bf16 and fp8).  The product's k index 8r + j (j < 4) is token 4r + j of the first
// sub-tile and 8r + 4 + j token 4r + j of the second, for both operands: lane l (r = l/16)
// holds, for its dim, the first sub-tile's V chunk half next to the second's, and the
// probabilities p0[j], p1[j] it already has from QK.
template <int KV, int D>
__device__ __forceinline__ void pv_pair(f32x4* acc, const uint4* vf0, const uint4* vf1, const float* p0,
                                        const float* p1) {
  if constexpr (KV == PKV_F32) {
    pv_subtile<KV, D>(acc, vf0, p0);
    pv_subtile<KV, D>(acc, vf1, p1);
  } else {
    const uint4 b = make_uint4(pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                               pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3]));
#pragma unroll
    for (int i = 0; i < Frag<KV, D>::NLOAD; ++i) {
      if constexpr (KV == PKV_BF16) {
        acc[2 * i + 0] = mfma_bf16_k32(make_uint4(vf0[i].x, vf0[i].y, vf1[i].x, vf1[i].y), b, acc[2 * i + 0]);
        acc[2 * i + 1] = mfma_bf16_k32(make_uint4(vf0[i].z, vf0[i].w, vf1[i].z, vf1[i].w), b, acc[2 * i + 1]);
      } else {
        const uint32_t w0[4] = {vf0[i].x, vf0[i].y, vf0[i].z, vf0[i].w};
        const uint32_t w1[4] = {vf1[i].x, vf1[i].y, vf1[i].z, vf1[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[4 * i + e] = mfma_bf16_k32(make_uint4(fp8x2_to_bf16x2<false>(w0[e]), fp8x2_to_bf16x2<true>(w0[e]),
                                                    fp8x2_to_bf16x2<false>(w1[e]), fp8x2_to_bf16x2<true>(w1[e])),
                                         b, acc[4 * i + e]);
      }
    }
  }
}

// Decoded value of an e4m3fn code (exact, through bf16).
__device__ __forceinline__ float e4m3fn_value(uint32_t code) {
  return __uint_as_float(fp8x2_to_bf16x2<false>(code) << 16);
}

}  // namespace tile
}  // namespace pkv
