// Exact top-K selection inside one workgroup.
//
// Result: the K largest candidate values, ties broken towards the lowest
// candidate position. The routine only finds the threshold: the K-th largest
// value T and `need`, the number of candidates equal to T that are kept
// (the first `need` of them in position order). The caller then keeps
// every candidate with value > T plus those first `need` ties, in position
// order, which yields ascending ids when positions are ordered by id.
//
// Algorithm (one workgroup, NT threads): a min/max pass; then up to
// kLevels rounds of a value-range histogram with NB linear bins over the
// current range [lo, hi] (LDS atomics); the bin holding the K-th largest
// value becomes the next range. Linear bins spread integer-valued and
// normally distributed scores over many bins, so the LDS atomics rarely
// collide. A range that collapses to one value ends the search; after
// kLevels rounds an exact bisection on order-preserving 32-bit keys finishes
// it. Float comparisons treat -0.0 and +0.0 as equal, as required.
#pragma once

#include "common.hpp"

namespace hisa {

template <int NT, int NB>
struct SelectLds {
  uint32_t hist[NB];
  uint32_t red[2 * (NT / kWave) + 2];
  float fred[2 * (NT / kWave) + 2];
  float thr;
  int need;
  int beta;
  uint32_t above;
};

struct Threshold {
  float T;    // values > T are kept
  int need;   // plus the first `need` values == T
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Get(c, i, v) loads item i (0 <= i < ITEMS) of this thread in chunk c into
// v and returns whether it is a valid candidate. Chunks are visited in
// order; thread t owns positions c*NT*ITEMS + t*ITEMS + i.
template <int NT, int ITEMS, int NB, class Get>
__device__ Threshold select_threshold(Get get, int nchunks, int K, SelectLds<NT, NB>& sh) {
  constexpr int kLevels = 3;
  static_assert(NB % NT == 0 || NT % NB == 0, "bins/threads");
  float mn = INFINITY, mx = -INFINITY;
  uint32_t cnt = 0;
  for (int c = 0; c < nchunks; ++c) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      float v;
      if (get(c, i, v)) {
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
        ++cnt;
      }
    }
  }
  const uint32_t n = block_sum<NT>(cnt, sh.red);
  block_minmax<NT>(mn, mx, sh.fred);
  if (n <= static_cast<uint32_t>(K)) return Threshold{-INFINITY, 0x7fffffff};
  float lo = mn, hi = mx;
  int krem = K;
  for (int level = 0; level < kLevels; ++level) {
    if (lo == hi) return Threshold{lo, krem};
    const float half_w = hi * 0.5f - lo * 0.5f;
    if (!(half_w > 0.0f)) break;
    const float scale = static_cast<float>(NB) / half_w;
    const float lo_h = lo * 0.5f;
    auto binof = [&](float v) {
      const int b = static_cast<int>((v * 0.5f - lo_h) * scale);
      return b < NB - 1 ? b : NB - 1;
    };
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += NT) sh.hist[b] = 0u;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        float v;
        if (get(c, i, v) && v >= lo && v <= hi) atomicAdd(&sh.hist[binof(v)], 1u);
      }
    }
    __syncthreads();
    // Suffix scan over the bins from the top: thread t owns reversed bins
    // r = t*BPT .. t*BPT+BPT-1 (bin NB-1-r).
    constexpr int BPT = NB >= NT ? NB / NT : 1;
    uint32_t local = 0;
    const bool owner = (threadIdx.x * BPT) < NB;
    if (owner) {
#pragma unroll
      for (int r = 0; r < BPT; ++r) local += sh.hist[NB - 1 - (threadIdx.x * BPT + r)];
    }
    uint32_t tot;
    uint32_t acc = block_excl_scan<NT>(local, tot, sh.red);
    if (owner) {
#pragma unroll
      for (int r = 0; r < BPT; ++r) {
        const int b = NB - 1 - (threadIdx.x * BPT + r);
        const uint32_t h = sh.hist[b];
        if (acc < static_cast<uint32_t>(krem) && acc + h >= static_cast<uint32_t>(krem)) {
          sh.beta = b;
          sh.above = acc;
        }
        acc += h;
      }
    }
    __syncthreads();
    const int beta = sh.beta;
    krem -= static_cast<int>(sh.above);
    float bmn = INFINITY, bmx = -INFINITY;
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        float v;
        if (get(c, i, v) && v >= lo && v <= hi && binof(v) == beta) {
          bmn = fminf(bmn, v);
          bmx = fmaxf(bmx, v);
        }
      }
    }
    block_minmax<NT>(bmn, bmx, sh.fred);
    lo = bmn;
    hi = bmx;
  }
  if (lo == hi) return Threshold{lo, krem};
  // Exact bisection on order keys within [lo, hi]: find the largest key x
  // with count(values in [x, hi]) >= krem.
  uint32_t klo = order_key(lo), khi = order_key(hi);
  while (klo < khi) {
    const uint32_t mid = klo + ((khi - klo + 1u) >> 1);
    const float fm = key_value(mid);
    uint32_t c2 = 0;
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        float v;
        if (get(c, i, v) && v >= fm && v <= hi) ++c2;
      }
    }
    const uint32_t tot = block_sum<NT>(c2, sh.red);
    if (tot >= static_cast<uint32_t>(krem)) klo = mid; else khi = mid - 1u;
  }
  const float T = key_value(klo);
  uint32_t gt = 0;
  for (int c = 0; c < nchunks; ++c) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      float v;
      if (get(c, i, v) && v > T && v <= hi) ++gt;
    }
  }
  const uint32_t tgt = block_sum<NT>(gt, sh.red);
  return Threshold{T, krem - static_cast<int>(tgt)};
}

// Position-ordered compaction of the kept candidates of one chunk. `base`
// carries (kept so far, ties seen so far) across chunks. Emit(pos, i, v) is
// called for every kept item i of this thread with its output position.
template <int NT, int ITEMS, int NB, class Get, class Emit>
__device__ void select_compact(Get get, int chunk, const Threshold th, uint32_t& kept_base,
                               uint32_t& tie_base, SelectLds<NT, NB>& sh, Emit emit) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    float v;
    if (get(chunk, i, v)) {
      gt += (v > th.T);
      eq += (v == th.T);
    }
  }
  // Pack (gt, eq) into one word: each count fits in 16 bits per chunk.
  uint32_t tot;
  const uint32_t pre = block_excl_scan<NT>((gt << 16) | eq, tot, sh.red);
  uint32_t ties = tie_base + (pre & 0xffffu);
  const uint32_t need = static_cast<uint32_t>(th.need);
  uint32_t pos = kept_base + (pre >> 16) + min(tie_base + (pre & 0xffffu), need) -
                 min(tie_base, need);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    float v;
    if (get(chunk, i, v)) {
      bool keep = v > th.T;
      if (v == th.T) {
        keep = ties < need;
        ++ties;
      }
      if (keep) emit(pos++, i, v);
    }
  }
  const uint32_t add_ties = tot & 0xffffu;
  kept_base += (tot >> 16) + min(tie_base + add_ties, need) - min(tie_base, need);
  tie_base += add_ties;
}

}  // namespace hisa
