// Two-level softmax decode (HiLS chapter, "hierarchical softmax
// decomposition": attention weight = inter-chunk share x intra-chunk share;
// HiLS-7B write-up: chunks are routed through compressed chunk keys, then
// fine attention runs inside the chosen chunks).
//
// One workgroup of W waves per (sequence, head) (16 for head width 64, 8 for
// 128, whose K and V registers are twice as many); wave w takes the chosen
// chunks w, w+W, ... For each 64-token group of a chunk, the K rows (lane =
// token) and the V values (lane = a pair of value columns and half of the
// tokens) are loaded together in one round trip. Lanes score their tokens
// (q . k_j in fp32, q broadcast from LDS), the wave forms the intra-chunk
// softmax over the tokens j <= t, and the value lanes accumulate
// sum_j p_j v_j; the two token halves meet through a lane-half swap. The
// chunk logit is scale_chunk * q . khat_c. A final pass takes the softmax
// over the chosen chunks' logits and mixes the chunk results a_c.
#include "common.hpp"
#include "internal.h"

namespace hisa {

template <int D, int W>
__global__ __launch_bounds__(64 * W) void hils_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const int32_t* __restrict__ chunk_idx, int L, int H, int C, int n_rows, int m,
    float scale_chunk, float scale_token, uint16_t* __restrict__ out, Str3 os) {
  constexpr int MAXM = 64;
  constexpr int NP = D / 2;        // value lanes per token (two columns each)
  constexpr int TH = 64 / NP;      // token halves per 64-token group (2 for D = 64)
  constexpr int TPL = 64 / TH;     // tokens per value lane per group
  constexpr int KV = D / 8;        // 16-byte pieces of a K row
  __shared__ float ac[MAXM][D];
  __shared__ float logit[MAXM];
  __shared__ __align__(16) float qf[D];
  __shared__ __align__(16) float pw[W][64];  // one group's numerators
  const int bh = blockIdx.x;  // b*H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int t = L - 1;
  for (int e = tid; e < D; e += 64 * W) qf[e] = bf16_to_f32(q[b * qs.b + h * qs.h + e]);
  __syncthreads();
  const int32_t* cidx = chunk_idx + static_cast<int64_t>(bh) * m;
  const uint16_t* kb = k + b * ks.b + h * ks.h;
  const uint16_t* vb = v + b * vs.b + h * vs.h;
  const int dp = lane % NP, th = lane / NP;
  float* pwv = pw[wave];
  for (int ci = wave; ci < m; ci += W) {
    const int c = cidx[ci];
    if (c < 0 || c >= n_rows) {
      if (lane == 0) logit[ci] = -INFINITY;
      continue;
    }
    // chunk logit
    const float* kh = khat + (static_cast<int64_t>(bh) * n_rows + c) * D;
    float part = 0.0f;
    for (int e = lane; e < D; e += kWave) part = fmaf(qf[e], kh[e], part);
    const float r = wave_sum(part) * scale_chunk;
    const int j0 = c * C, j1 = min(min(L, j0 + C), t + 1);  // j0 <= t: one valid token at least
    // one pass over the chunk's 64-token groups with a running maximum: the
    // K rows (lane = token) and the V values (lane (dp, th): columns 2dp,
    // 2dp+1 of tokens TPL*th + i) of a group are loaded together
    float mrun = -INFINITY, lsum = 0.0f, a0 = 0.0f, a1 = 0.0f;
    for (int g0 = j0; g0 < j1; g0 += 64) {
      const int j = g0 + lane;
      const int jb = g0 + TPL * th;
      uint4 kw[KV];
      uint32_t vw[TPL];
      if (j < j1) {
        const uint16_t* kr = kb + static_cast<int64_t>(j) * ks.t;
#pragma unroll
        for (int x = 0; x < KV; ++x) kw[x] = *reinterpret_cast<const uint4*>(kr + 8 * x);
      }
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        vw[i] = jb + i < j1 ? *reinterpret_cast<const uint32_t*>(
                                  vb + static_cast<int64_t>(jb + i) * vs.t + 2 * dp)
                            : 0u;
      float s = -INFINITY;
      if (j < j1) {
        float acc = 0.0f;
#pragma unroll
        for (int x = 0; x < KV; ++x) {
          const float4 qa = *reinterpret_cast<const float4*>(&qf[8 * x]);
          const float4 qb = *reinterpret_cast<const float4*>(&qf[8 * x + 4]);
          acc = fmaf(qa.x, bf16_lo(kw[x].x), acc); acc = fmaf(qa.y, bf16_hi(kw[x].x), acc);
          acc = fmaf(qa.z, bf16_lo(kw[x].y), acc); acc = fmaf(qa.w, bf16_hi(kw[x].y), acc);
          acc = fmaf(qb.x, bf16_lo(kw[x].z), acc); acc = fmaf(qb.y, bf16_hi(kw[x].z), acc);
          acc = fmaf(qb.z, bf16_lo(kw[x].w), acc); acc = fmaf(qb.w, bf16_hi(kw[x].w), acc);
        }
        s = acc * scale_token;
      }
      const float mnew = fmaxf(mrun, wave_max(s));  // finite: the group has a valid token
      const float f = mrun == -INFINITY ? 0.0f : __expf(mrun - mnew);
      const float p = j < j1 ? __expf(s - mnew) : 0.0f;
      lsum = lsum * f + p;
      a0 *= f;
      a1 *= f;
      mrun = mnew;
      pwv[lane] = p;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      const float* pp = pwv + TPL * th;
#pragma unroll
      for (int i = 0; i < TPL; i += 4) {
        const float4 p4 = *reinterpret_cast<const float4*>(pp + i);
        a0 = fmaf(p4.x, bf16_lo(vw[i + 0]), a0); a1 = fmaf(p4.x, bf16_hi(vw[i + 0]), a1);
        a0 = fmaf(p4.y, bf16_lo(vw[i + 1]), a0); a1 = fmaf(p4.y, bf16_hi(vw[i + 1]), a1);
        a0 = fmaf(p4.z, bf16_lo(vw[i + 2]), a0); a1 = fmaf(p4.z, bf16_hi(vw[i + 2]), a1);
        a0 = fmaf(p4.w, bf16_lo(vw[i + 3]), a0); a1 = fmaf(p4.w, bf16_hi(vw[i + 3]), a1);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    }
    const float sum = wave_sum(lsum);
    if constexpr (TH == 2) {
      // the other token half sits in lane l ^ 32
      const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a0),
                                                       false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a1), __float_as_uint(a1),
                                                       false, false);
      a0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
      a1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
    }
    if (th == 0) {
      ac[ci][2 * dp] = a0 / sum;
      ac[ci][2 * dp + 1] = a1 / sum;
    }
    if (lane == 0) logit[ci] = r;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
  __syncthreads();
  for (int e = tid; e < D; e += 64 * W) {
    float mx = -INFINITY;
    for (int ci = 0; ci < m; ++ci) mx = fmaxf(mx, logit[ci]);
    float z = 0.0f, acc = 0.0f;
    for (int ci = 0; ci < m; ++ci) {
      if (logit[ci] == -INFINITY) continue;
      const float w = __expf(logit[ci] - mx);
      z += w;
      acc = fmaf(w, ac[ci][e], acc);
    }
    out[b * os.b + h * os.h + e] = f32_to_bf16(z > 0.0f ? acc / z : 0.0f);
  }
}

hipError_t launch_hils(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks, const uint16_t* v,
                       Str3 vs, const float* khat, const int32_t* chunk_idx, int batch, int L,
                       int H, int D, int C, int n_rows, int m, float scale_chunk,
                       float scale_token, uint16_t* out, Str3 os, hipStream_t s) {
  dim3 grid(batch * H);
  if (D == 64)
    hipLaunchKernelGGL((hils_kernel<64, 16>), grid, dim3(64 * 16), 0, s, q, qs, k, ks, v, vs,
                       khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  else
    hipLaunchKernelGGL((hils_kernel<128, 8>), grid, dim3(64 * 8), 0, s, q, qs, k, ks, v, vs,
                       khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  return hipGetLastError();
}

}  // namespace hisa
