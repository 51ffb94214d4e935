// Device helpers shared by the gfx950 kernels: bf16 packing, matrix-core
// (MFMA) fragments, wavefront reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hisa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits: the hardware conversion
// (v_cvt_pk_bf16_f32, two values per instruction; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l holds A row (l % 16) and B column (l % 16), each with 8 consecutive
// k values of group (l / 16); D lane l holds column (l % 16), rows
// 4*(l/16) .. 4*(l/16)+3. Any consistent assignment of data to k slots gives
// the same contraction, which the kernels use to pick convenient layouts.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- waves
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t u = __shfl_up(v, o, kWave);
    if (l >= o) v += u;
  }
  return v;
}

// The same through the VALU's data-parallel lane moves (DPP): shifts within
// 16-lane rows, then the row broadcasts of lanes 15 and 31. No LDS traffic;
// the result of a reduction is complete in lane 63.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(v), CTRL, ROWMASK, 0xf, false));
}
// inclusive prefix sum across the 64 lanes
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
  v += dpp_move<0x111, 0xf>(0u, v);  // row_shr:1
  v += dpp_move<0x112, 0xf>(0u, v);  // row_shr:2
  v += dpp_move<0x114, 0xf>(0u, v);  // row_shr:4
  v += dpp_move<0x118, 0xf>(0u, v);  // row_shr:8
  v += dpp_move<0x142, 0xa>(0u, v);  // row_bcast:15 into rows 1, 3
  v += dpp_move<0x143, 0xc>(0u, v);  // row_bcast:31 into rows 2, 3
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_scan_dpp(v)), 63));
}
// maximum / minimum across the 64 lanes (NaN lanes are ignored, as fmaxf does)
template <bool MAX>
__device__ __forceinline__ float wave_ext_dpp(float x) {
  auto step = [&](uint32_t moved) {
    const float o = __uint_as_float(moved);
    x = MAX ? fmaxf(x, o) : fminf(x, o);
  };
  step(dpp_move<0x111, 0xf>(__float_as_uint(x), __float_as_uint(x)));
  step(dpp_move<0x112, 0xf>(__float_as_uint(x), __float_as_uint(x)));
  step(dpp_move<0x114, 0xf>(__float_as_uint(x), __float_as_uint(x)));
  step(dpp_move<0x118, 0xf>(__float_as_uint(x), __float_as_uint(x)));
  step(dpp_move<0x142, 0xa>(__float_as_uint(x), __float_as_uint(x)));
  step(dpp_move<0x143, 0xc>(__float_as_uint(x), __float_as_uint(x)));
  return __uint_as_float(
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(x)), 63)));
}
// minimum of an unsigned value across the 64 lanes, the same for every lane
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_move<0x111, 0xf>(x, x));  // row_shr:1
  x = min(x, dpp_move<0x112, 0xf>(x, x));  // row_shr:2
  x = min(x, dpp_move<0x114, 0xf>(x, x));  // row_shr:4
  x = min(x, dpp_move<0x118, 0xf>(x, x));  // row_shr:8
  x = min(x, dpp_move<0x142, 0xa>(x, x));  // row_bcast:15 into rows 1, 3
  x = min(x, dpp_move<0x143, 0xc>(x, x));  // row_bcast:31 into rows 2, 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
// maximum of an unsigned value across the 64 lanes, the same for every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_move<0x111, 0xf>(x, x));  // row_shr:1
  x = max(x, dpp_move<0x112, 0xf>(x, x));  // row_shr:2
  x = max(x, dpp_move<0x114, 0xf>(x, x));  // row_shr:4
  x = max(x, dpp_move<0x118, 0xf>(x, x));  // row_shr:8
  x = max(x, dpp_move<0x142, 0xa>(x, x));  // row_bcast:15 into rows 1, 3
  x = max(x, dpp_move<0x143, 0xc>(x, x));  // row_bcast:31 into rows 2, 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
// number of set bits of `mask` in the lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Block-wide reductions over NT threads; `red` is LDS scratch of >= NT/64
// words. Every thread of the block must call them (they synchronise).
template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* red) {
  v = wave_sum(v);
  if constexpr (NT == kWave) {
    return v;
  } else {
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if (lane_id() == 0) red[w] = v;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) s += red[i];
    return s;
  }
}
template <int NT>
__device__ __forceinline__ void block_minmax(float& mn, float& mx, float* red) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  if constexpr (NT != kWave) {
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if (lane_id() == 0) {
      red[2 * w] = mn;
      red[2 * w + 1] = mx;
    }
    __syncthreads();
    mn = red[0];
    mx = red[1];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) {
      mn = fminf(mn, red[2 * i]);
      mx = fmaxf(mx, red[2 * i + 1]);
    }
  }
}
// Block-wide exclusive scan; returns the exclusive prefix, `total` the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, uint32_t* red) {
  uint32_t inc = wave_incl_scan(v);
  if constexpr (NT == kWave) {
    total = __shfl(inc, kWave - 1, kWave);
    return inc - v;
  } else {
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if (lane_id() == kWave - 1) red[w] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
      const uint32_t r = red[i];
      before += (i < w) ? r : 0u;
      all += r;
    }
    total = all;
    return before + inc - v;
  }
}

}  // namespace hisa
