// Two-level softmax decode (HiLS chapter, "hierarchical softmax
// decomposition": attention weight = inter-chunk share x intra-chunk share;
// HiLS-7B write-up: chunks are routed through compressed chunk keys, then
// fine attention runs inside the chosen chunks).
//
// One workgroup per (sequence, head), one wave per chosen chunk at a time:
// lanes score the chunk's tokens (q . k_j, fp32), the wave forms the
// intra-chunk softmax and its weighted value sum a_c through LDS, and the
// chunk logit is scale_chunk * q . khat_c. A final pass takes the softmax
// over the chosen chunks' logits and mixes the a_c.
#include "common.hpp"
#include "internal.h"

namespace hisa {

template <int D>
__global__ __launch_bounds__(256) void hils_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const int32_t* __restrict__ chunk_idx, int L, int H, int C, int n_rows, int m,
    float scale_chunk, float scale_token, uint16_t* __restrict__ out, Str3 os) {
  constexpr int MAXM = 64, MAXC = 256;
  __shared__ float ac[MAXM][D];
  __shared__ float logit[MAXM];
  __shared__ float qf[D];
  __shared__ float pw[4][MAXC];
  const int bh = blockIdx.x;  // b*H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int t = L - 1;
  for (int e = tid; e < D; e += 256) qf[e] = bf16_to_f32(q[b * qs.b + h * qs.h + e]);
  __syncthreads();
  const int32_t* cidx = chunk_idx + static_cast<int64_t>(bh) * m;
  for (int ci = wave; ci < m; ci += 4) {
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
    // token scores: lane handles tokens j = c*C + lane + 64*i
    const int j0 = c * C, j1 = min(min(L, j0 + C), t + 1);
    float mx = -INFINITY;
    for (int j = j0 + lane; j < j1; j += kWave) {
      const uint16_t* kr = k + b * ks.b + static_cast<int64_t>(j) * ks.t + h * ks.h;
      float s = 0.0f;
      for (int e = 0; e < D; e += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(kr + e);
        s = fmaf(qf[e + 0], bf16_lo(w.x), s); s = fmaf(qf[e + 1], bf16_hi(w.x), s);
        s = fmaf(qf[e + 2], bf16_lo(w.y), s); s = fmaf(qf[e + 3], bf16_hi(w.y), s);
        s = fmaf(qf[e + 4], bf16_lo(w.z), s); s = fmaf(qf[e + 5], bf16_hi(w.z), s);
        s = fmaf(qf[e + 6], bf16_lo(w.w), s); s = fmaf(qf[e + 7], bf16_hi(w.w), s);
      }
      s *= scale_token;
      pw[wave][j - j0] = s;
      mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int j = j0 + lane; j < j1; j += kWave) {
      const float p = __expf(pw[wave][j - j0] - mx);
      pw[wave][j - j0] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    // a_c[e] = sum_j p_j v_j[e] / sum; lane owns dims e = lane + 64*i
    for (int e = lane; e < D; e += kWave) {
      float a = 0.0f;
      for (int j = j0; j < j1; ++j)
        a = fmaf(pw[wave][j - j0],
                 bf16_to_f32(v[b * vs.b + static_cast<int64_t>(j) * vs.t + h * vs.h + e]), a);
      ac[ci][e] = a / sum;
    }
    if (lane == 0) logit[ci] = r;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
  __syncthreads();
  for (int e = tid; e < D; e += 256) {
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
    hipLaunchKernelGGL(hils_kernel<64>, grid, dim3(256), 0, s, q, qs, k, ks, v, vs, khat,
                       chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  else
    hipLaunchKernelGGL(hils_kernel<128>, grid, dim3(256), 0, s, q, qs, k, ks, v, vs, khat,
                       chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  return hipGetLastError();
}

}  // namespace hisa
