// Sparse attention over the selected tokens (HISA explainer 1.1: attention
// only between a query and its selected key tokens; HISA news article: the
// downstream sparse attention is unchanged by the hierarchical indexer).
//
// One workgroup per (sequence, query, kv head): the GP (>= heads in the
// group, padded to a multiple of 16) query heads that share one kv head form
// the M dimension of both matrix-core products. Each tile of NT selected
// tokens is gathered from HBM into LDS (K row-major, V transposed so both
// products read contiguous 16-byte fragments), S = Q K^T runs on the bf16
// matrix cores, an online softmax (base-2 exponent, fp32) updates the row
// statistics, and O += P V accumulates in registers.
#include "common.hpp"
#include "internal.h"

namespace hisa {

template <int GP, int DK, int DV, bool VALIAS>
struct AttnLds {
  static constexpr int NT = 32;
  static constexpr int QLD = DK + 8;  // padded row (bf16 elements)
  uint16_t q[GP * QLD];
  uint16_t k[NT * QLD];
  uint16_t vt[DV * NT];
  uint16_t p[GP * NT];
  float s[GP * NT];
  float alpha[GP];
  float lrow[GP];
  float mrow[GP];
  int tok[NT];
};

template <int GP, int DK, int DV, bool VALIAS>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, int nq, int L, int G,
    const int32_t* __restrict__ token_idx, int topk, float scale_log2, uint16_t* __restrict__ out,
    Str3 os, float* __restrict__ lse) {
  using Lds = AttnLds<GP, DK, DV, VALIAS>;
  constexpr int NT = Lds::NT, QLD = Lds::QLD;
  constexpr int MT = GP / 16;
  constexpr int NOT = DV / 16;               // output column tiles
  constexpr int OT_PER_WAVE = (MT * NOT) / 4;
  static_assert((MT * NOT) % 4 == 0, "output tiles must split over 4 waves");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Lds& sh = *reinterpret_cast<Lds*>(smem_raw);

  const int qi = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lg = lane / 16, r16 = lane % 16;
  const int64_t qrow = static_cast<int64_t>(b) * nq + qi;
  const int32_t* tix = token_idx + qrow * topk;

  // Q rows of this group into LDS (rows >= G zero)
  for (int e = tid; e < GP * (DK / 8); e += 256) {
    const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < G)
      val = *reinterpret_cast<const uint4*>(q + b * qs.b + qi * qs.t + (g * G + r) * qs.h + cc);
    *reinterpret_cast<uint4*>(&sh.q[r * QLD + cc]) = val;
  }
  if (tid < GP) {
    sh.mrow[tid] = -INFINITY;
    sh.lrow[tid] = 0.0f;
  }
  f32x4 o[OT_PER_WAVE];
#pragma unroll
  for (int i = 0; i < OT_PER_WAVE; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const uint16_t* kb = k + b * ks.b + g * ks.h;
  const uint16_t* vb = v + b * vs.b + g * vs.h;
  for (int t0 = 0; t0 < topk; t0 += NT) {
    __syncthreads();
    if (tid < NT) {
      const int j = t0 + tid < topk ? tix[t0 + tid] : -1;
      sh.tok[tid] = j < L ? j : -1;
    }
    __syncthreads();
    // gather K rows (and V, transposed)
    for (int e = tid; e < NT * (DK / 8); e += 256) {
      const int r = e / (DK / 8), cc = (e % (DK / 8)) * 8;
      const int j = sh.tok[r];
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j >= 0) val = *reinterpret_cast<const uint4*>(kb + j * ks.t + cc);
      *reinterpret_cast<uint4*>(&sh.k[r * QLD + cc]) = val;
      if constexpr (VALIAS) {
        if (cc < DV) {
          const uint16_t* pv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
          for (int x = 0; x < 8; ++x) sh.vt[(cc + x) * NT + r] = pv[x];
        }
      }
    }
    if constexpr (!VALIAS) {
      for (int e = tid; e < NT * (DV / 8); e += 256) {
        const int r = e / (DV / 8), cc = (e % (DV / 8)) * 8;
        const int j = sh.tok[r];
        uint4 val = make_uint4(0, 0, 0, 0);
        if (j >= 0) val = *reinterpret_cast<const uint4*>(vb + j * vs.t + cc);
        const uint16_t* pv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
        for (int x = 0; x < 8; ++x) sh.vt[(cc + x) * NT + r] = pv[x];
      }
    }
    __syncthreads();
    // S = Q K^T, tiles (mt, nt) with nt in {0, 1}
    for (int tt = wave; tt < MT * 2; tt += 4) {
      const int mt = tt / 2, nt = tt % 2;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* qa = &sh.q[(mt * 16 + r16) * QLD + 8 * lg];
      const uint16_t* kbp = &sh.k[(nt * 16 + r16) * QLD + 8 * lg];
#pragma unroll 6
      for (int s = 0; s < DK / 32; ++s)
        acc = mfma16(as_bf16x8(*reinterpret_cast<const uint4*>(qa + 32 * s)),
                     as_bf16x8(*reinterpret_cast<const uint4*>(kbp + 32 * s)), acc);
      const int col = nt * 16 + r16;
      const bool live = sh.tok[col] >= 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sh.s[(mt * 16 + 4 * lg + r) * NT + col] = live ? acc[r] * scale_log2 : -INFINITY;
    }
    __syncthreads();
    // online softmax, one thread per row
    if (tid < GP) {
      const float* sr = &sh.s[tid * NT];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NT; ++j) mx = fmaxf(mx, sr[j]);
      const float mold = sh.mrow[tid];
      const float mnew = fmaxf(mold, mx);
      float alpha = 1.0f, sum = 0.0f;
      if (mnew == -INFINITY) {
#pragma unroll
        for (int j = 0; j < NT; ++j) sh.p[tid * NT + j] = 0;
      } else {
        alpha = exp2f(mold - mnew);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const uint16_t pb = f32_to_bf16(exp2f(sr[j] - mnew));
          sh.p[tid * NT + j] = pb;
          sum += bf16_to_f32(pb);
        }
      }
      sh.alpha[tid] = alpha;
      sh.mrow[tid] = mnew;
      sh.lrow[tid] = sh.lrow[tid] * alpha + sum;
    }
    __syncthreads();
    // O = alpha * O + P V
#pragma unroll
    for (int i = 0; i < OT_PER_WAVE; ++i) {
      const int ot = wave * OT_PER_WAVE + i;
      const int mt = ot / NOT, nt = ot % NOT;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[i][r] *= sh.alpha[mt * 16 + 4 * lg + r];
      const bf16x8 pa = as_bf16x8(*reinterpret_cast<const uint4*>(&sh.p[(mt * 16 + r16) * NT + 8 * lg]));
      const bf16x8 vbf = as_bf16x8(*reinterpret_cast<const uint4*>(&sh.vt[(nt * 16 + r16) * NT + 8 * lg]));
      o[i] = mfma16(pa, vbf, o[i]);
    }
  }
  __syncthreads();
  // normalise and store
#pragma unroll
  for (int i = 0; i < OT_PER_WAVE; ++i) {
    const int ot = wave * OT_PER_WAVE + i;
    const int mt = ot / NOT, nt = ot % NOT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * lg + r;
      if (row < G) {
        const float l = sh.lrow[row];
        const float val = l > 0.0f ? o[i][r] / l : 0.0f;
        out[b * os.b + qi * os.t + (g * G + row) * os.h + nt * 16 + r16] = f32_to_bf16(val);
      }
    }
  }
  if (lse != nullptr && tid < G) {
    const float l = sh.lrow[tid];
    lse[qrow * (static_cast<int64_t>(G) * gridDim.y) + g * G + tid] =
        l > 0.0f ? (sh.mrow[tid] + log2f(l)) * 0.69314718055994530942f : -INFINITY;
  }
}

template <int GP, int DK, int DV, bool VALIAS>
static hipError_t attn_launch(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                              const uint16_t* v, Str3 vs, int batch, int nq, int L, int Hkv, int G,
                              const int32_t* tix, int topk, float scale, uint16_t* out, Str3 os,
                              float* lse, hipStream_t s) {
  const size_t lds = sizeof(AttnLds<GP, DK, DV, VALIAS>);
  auto kern = sparse_attn_kernel<GP, DK, DV, VALIAS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.44269504088896340736f;
  hipLaunchKernelGGL(kern, dim3(nq, Hkv, batch), dim3(256), lds, s, q, qs, k, ks, v, vs, nq, L, G,
                     tix, topk, scale_log2, out, os, lse);
  return hipGetLastError();
}

// Only the head-width-128 kernel uses a workspace (the split of few long
// token lists).
size_t sparse_attn_workspace(int batch, int nq, int Hq, int Hkv, int Dk, int Dv, int topk) {
  const int G = Hq / Hkv;
  if (Dk == 128 && Dv == 128 && G <= 16) return attn_d128_workspace(batch, nq, Hkv, G, topk);
  return 0;
}

hipError_t launch_sparse_attn(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                              const uint16_t* v, Str3 vs, int batch, int nq, int L, int Hq,
                              int Hkv, int Dk, int Dv, const int32_t* token_idx, int topk,
                              float scale, uint16_t* out, Str3 os, float* lse, void* ws,
                              hipStream_t s) {
  const int G = Hq / Hkv;
  const bool alias = (v == k) && vs.b == ks.b && vs.t == ks.t && vs.h == ks.h;
#define HISA_ATT(GP_, DK_, DV_, AL_) \
  return attn_launch<GP_, DK_, DV_, AL_>(q, qs, k, ks, v, vs, batch, nq, L, Hkv, G, token_idx, \
                                         topk, scale, out, os, lse, s)
  if (Dk == 576 && alias && G == 64)
    return launch_mla_attn(q, qs, k, ks, batch, nq, L, Hkv, token_idx, topk, scale, out, os, lse, s);
  if (Dk == 128 && Dv == 128 && G <= 16)
    return launch_attn_d128(q, qs, k, ks, v, vs, batch, nq, L, Hkv, G, token_idx, topk, scale, out,
                            os, lse, ws, s);
  if (Dk == 576) {
    if (alias) {
      if (G <= 16) HISA_ATT(16, 576, 512, true);
      if (G <= 32) HISA_ATT(32, 576, 512, true);
      HISA_ATT(64, 576, 512, true);
    } else {
      if (G <= 16) HISA_ATT(16, 576, 512, false);
      if (G <= 32) HISA_ATT(32, 576, 512, false);
      HISA_ATT(64, 576, 512, false);
    }
  } else if (Dk == 128) {
    if (G <= 16) HISA_ATT(16, 128, 128, false);
    if (G <= 32) HISA_ATT(32, 128, 128, false);
    HISA_ATT(64, 128, 128, false);
  } else {
    if (G <= 16) HISA_ATT(16, 64, 64, false);
    if (G <= 32) HISA_ATT(32, 64, 64, false);
    HISA_ATT(64, 64, 64, false);
  }
#undef HISA_ATT
}

}  // namespace hisa
