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
//
// With a workspace and few (sequence, head) pairs, the chosen chunks are
// spread over many workgroups instead (four waves, one chunk each), which
// write a_c and the chunk logits; a second kernel mixes them per pair. One
// workgroup per pair would keep the whole step on as many CUs as there are
// pairs (16 at batch 1), each moving all 32 chunks through its own loads.
#include "common.hpp"
#include "internal.h"

namespace hisa {

// The chunk result of one wave: a_c (columns 2dp, 2dp+1 of it in the lanes
// of the first token half) and the chunk logit r_c.
template <int D>
struct ChunkOut {
  float a0, a1, r;
};

template <int D>
__device__ __forceinline__ ChunkOut<D> hils_chunk(const float* qf, const uint16_t* kb, int64_t kst,
                                                  const uint16_t* vb, int64_t vst, const float* kh,
                                                  int c, int C, int L, int t, float scale_chunk,
                                                  float scale_token, float* pwv, int lane) {
  constexpr int NP = D / 2;        // value lanes per token (two columns each)
  constexpr int TH = 64 / NP;      // token halves per 64-token group (2 for D = 64)
  constexpr int TPL = 64 / TH;     // tokens per value lane per group
  constexpr int KV = D / 8;        // 16-byte pieces of a K row
  const int dp = lane % NP, th = lane / NP;
  // the chunk key is loaded now and its product with q formed after the
  // chunk's token loads are issued
  float khv[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) khv[x] = kh[lane + 64 * x];
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
      const uint16_t* kr = kb + static_cast<int64_t>(j) * kst;
#pragma unroll
      for (int x = 0; x < KV; ++x) kw[x] = *reinterpret_cast<const uint4*>(kr + 8 * x);
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i)
      vw[i] = jb + i < j1 ? *reinterpret_cast<const uint32_t*>(
                                vb + static_cast<int64_t>(jb + i) * vst + 2 * dp)
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
  float part = 0.0f;
#pragma unroll
  for (int x = 0; x < D / 64; ++x) part = fmaf(qf[lane + 64 * x], khv[x], part);
  const float r = wave_sum(part) * scale_chunk;
  if constexpr (TH == 2) {
    // the other token half sits in lane l ^ 32
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a0),
                                                     false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a1), __float_as_uint(a1),
                                                     false, false);
    a0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
    a1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
  }
  return ChunkOut<D>{a0 / sum, a1 / sum, r};
}

// the softmax over the chosen chunks' logits, mixing their results
template <int D>
__device__ __forceinline__ float hils_mix(const float* logit, const float* ac, int m, int e) {
  float mx = -INFINITY;
  for (int ci = 0; ci < m; ++ci) mx = fmaxf(mx, logit[ci]);
  float z = 0.0f, acc = 0.0f;
  for (int ci = 0; ci < m; ++ci) {
    if (logit[ci] == -INFINITY) continue;
    const float w = __expf(logit[ci] - mx);
    z += w;
    acc = fmaf(w, ac[ci * D + e], acc);
  }
  return z > 0.0f ? acc / z : 0.0f;
}

template <int D, int W>
__global__ __launch_bounds__(64 * W) void hils_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const int32_t* __restrict__ chunk_idx, int L, int H, int C, int n_rows, int m,
    float scale_chunk, float scale_token, uint16_t* __restrict__ out, Str3 os) {
  constexpr int MAXM = 64;
  constexpr int NP = D / 2;
  __shared__ float ac[MAXM * D];
  __shared__ float logit[MAXM];
  __shared__ __align__(16) float qf[D];
  __shared__ __align__(16) float pw[W][64];  // one group's numerators
  const int bh = blockIdx.x;  // b*H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  for (int e = tid; e < D; e += 64 * W) qf[e] = bf16_to_f32(q[b * qs.b + h * qs.h + e]);
  __syncthreads();
  const int32_t* cidx = chunk_idx + static_cast<int64_t>(bh) * m;
  const uint16_t* kb = k + b * ks.b + h * ks.h;
  const uint16_t* vb = v + b * vs.b + h * vs.h;
  // this wave's chunk ids, read at once: lane i holds chunk wave + W*i
  const int nmine = (m - wave + W - 1) / W;
  const int cid = lane < nmine ? cidx[wave + W * lane] : -1;
  for (int it = 0; it < nmine; ++it) {
    const int ci = wave + W * it;
    const int c = __builtin_amdgcn_readlane(cid, it);
    if (c < 0 || c >= n_rows) {
      if (lane == 0) logit[ci] = -INFINITY;
      continue;
    }
    const ChunkOut<D> co =
        hils_chunk<D>(qf, kb, ks.t, vb, vs.t, khat + (static_cast<int64_t>(bh) * n_rows + c) * D,
                      c, C, L, L - 1, scale_chunk, scale_token, pw[wave], lane);
    if (lane < NP) {
      ac[ci * D + 2 * lane] = co.a0;
      ac[ci * D + 2 * lane + 1] = co.a1;
    }
    if (lane == 0) logit[ci] = co.r;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
  __syncthreads();
  for (int e = tid; e < D; e += 64 * W)
    out[b * os.b + h * os.h + e] = f32_to_bf16(hils_mix<D>(logit, ac, m, e));
}

// Causal two-level prefill: one workgroup of W waves per (sequence, head,
// query). The query at position t routes and attends as the decode of the
// first t+1 tokens: complete chunks keep their table keys, and the local
// chunk t / C is keyed by the projected mean of its tokens <= t, formed here
// (column sums split over the waves, then the projection).
template <int D, int W>
__global__ __launch_bounds__(64 * W) void hils_prefill_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const int32_t* __restrict__ chunk_idx, const uint16_t* __restrict__ proj,
    const int32_t* __restrict__ q_pos, int nq, int L, int H, int C, int n_rows, int m,
    float scale_chunk, float scale_token, uint16_t* __restrict__ out, Str3 os) {
  constexpr int MAXM = 64;
  constexpr int NP = D / 2;
  __shared__ float ac[MAXM * D];
  __shared__ float logit[MAXM];
  __shared__ __align__(16) float qf[D];
  __shared__ float kloc[D];        // the local chunk's key
  __shared__ float psum[W][D];     // per-wave column sums of the local chunk
  __shared__ __align__(16) float pw[W][64];
  const int qi = blockIdx.x;       // query of the sequence
  const int bh = blockIdx.y;       // b*H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int t = min(max(q_pos[static_cast<int64_t>(b) * nq + qi], 0), L - 1);
  const int bt = t / C;
  const uint16_t* kb = k + b * ks.b + h * ks.h;
  const uint16_t* vb = v + b * vs.b + h * vs.h;
  for (int e = tid; e < D; e += 64 * W)
    qf[e] = bf16_to_f32(q[b * qs.b + static_cast<int64_t>(qi) * qs.t + h * qs.h + e]);
#pragma unroll
  for (int x = 0; x < D / 64; ++x) {
    float acc = 0.0f;
    for (int j = bt * C + wave; j <= t; j += W)
      acc += bf16_to_f32(kb[static_cast<int64_t>(j) * ks.t + lane + 64 * x]);
    psum[wave][lane + 64 * x] = acc;
  }
  __syncthreads();
  for (int e = tid; e < D; e += 64 * W) {
    float pr = 0.0f;
    if (proj == nullptr) {
#pragma unroll
      for (int w = 0; w < W; ++w) pr += psum[w][e];
    } else {
      for (int d = 0; d < D; ++d) {
        float sd = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) sd += psum[w][d];
        pr = fmaf(bf16_to_f32(proj[e * D + d]), sd, pr);
      }
    }
    kloc[e] = pr / static_cast<float>(t - bt * C + 1);
  }
  __syncthreads();
  const int32_t* cidx = chunk_idx + (static_cast<int64_t>(bh) * nq + qi) * m;
  const int nmine = (m - wave + W - 1) / W;
  const int cid = lane < nmine ? cidx[wave + W * lane] : -1;
  for (int it = 0; it < nmine; ++it) {
    const int ci = wave + W * it;
    const int c = __builtin_amdgcn_readlane(cid, it);
    if (c < 0 || c > bt) {
      if (lane == 0) logit[ci] = -INFINITY;
      continue;
    }
    const float* kh = c == bt ? kloc : khat + (static_cast<int64_t>(bh) * n_rows + c) * D;
    const ChunkOut<D> co = hils_chunk<D>(qf, kb, ks.t, vb, vs.t, kh, c, C, L, t, scale_chunk,
                                         scale_token, pw[wave], lane);
    if (lane < NP) {
      ac[ci * D + 2 * lane] = co.a0;
      ac[ci * D + 2 * lane + 1] = co.a1;
    }
    if (lane == 0) logit[ci] = co.r;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
  __syncthreads();
  for (int e = tid; e < D; e += 64 * W)
    out[b * os.b + static_cast<int64_t>(qi) * os.t + h * os.h + e] =
        f32_to_bf16(hils_mix<D>(logit, ac, m, e));
}

hipError_t launch_hils_prefill(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                               const uint16_t* v, Str3 vs, const float* khat,
                               const int32_t* chunk_idx, const uint16_t* proj,
                               const int32_t* q_pos, int batch, int nq, int L, int H, int D,
                               int C, int n_rows, int m, float scale_chunk, float scale_token,
                               uint16_t* out, Str3 os, hipStream_t s) {
  const dim3 grid(nq, batch * H);
  if (D == 64)
    hipLaunchKernelGGL((hils_prefill_kernel<64, 16>), grid, dim3(64 * 16), 0, s, q, qs, k, ks, v,
                       vs, khat, chunk_idx, proj, q_pos, nq, L, H, C, n_rows, m, scale_chunk,
                       scale_token, out, os);
  else
    hipLaunchKernelGGL((hils_prefill_kernel<128, 8>), grid, dim3(64 * 8), 0, s, q, qs, k, ks, v,
                       vs, khat, chunk_idx, proj, q_pos, nq, L, H, C, n_rows, m, scale_chunk,
                       scale_token, out, os);
  return hipGetLastError();
}

// Split form, first kernel: workgroup (pair bh, chunks 4y .. 4y+3), one wave
// per chosen chunk; a_c into ws_a [pairs][m][D], the logit into ws_r [pairs][m].
template <int D>
__global__ __launch_bounds__(256) void hils_chunks_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const int32_t* __restrict__ chunk_idx, int L, int H, int C, int n_rows, int m,
    float scale_chunk, float scale_token, float* __restrict__ ws_a, float* __restrict__ ws_r) {
  constexpr int NP = D / 2;
  __shared__ __align__(16) float qf[D];
  __shared__ __align__(16) float pw[4][64];
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  for (int e = tid; e < D; e += 256) qf[e] = bf16_to_f32(q[b * qs.b + h * qs.h + e]);
  __syncthreads();
  const int ci = blockIdx.y * 4 + wave;
  if (ci >= m) return;
  const int c = chunk_idx[static_cast<int64_t>(bh) * m + ci];
  const int64_t slot = static_cast<int64_t>(bh) * m + ci;
  if (c < 0 || c >= n_rows) {
    if (lane == 0) ws_r[slot] = -INFINITY;
    return;
  }
  const ChunkOut<D> co = hils_chunk<D>(qf, k + b * ks.b + h * ks.h, ks.t, v + b * vs.b + h * vs.h,
                                       vs.t, khat + (static_cast<int64_t>(bh) * n_rows + c) * D,
                                       c, C, L, L - 1, scale_chunk, scale_token, pw[wave], lane);
  if (lane < NP)
    *reinterpret_cast<float2*>(ws_a + slot * D + 2 * lane) = make_float2(co.a0, co.a1);
  if (lane == 0) ws_r[slot] = co.r;
}

// Split form, second kernel: one workgroup per pair, one thread per column.
template <int D>
__global__ __launch_bounds__(D) void hils_merge_kernel(const float* __restrict__ ws_a,
                                                       const float* __restrict__ ws_r, int H,
                                                       int m, uint16_t* __restrict__ out,
                                                       Str3 os) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int64_t base = static_cast<int64_t>(bh) * m;
  out[b * os.b + h * os.h + threadIdx.x] =
      f32_to_bf16(hils_mix<D>(ws_r + base, ws_a + base * D, m, threadIdx.x));
}

// the split form pays while the pairs leave most CUs idle
constexpr int64_t kHilsSplitPairs = 256;

size_t hils_workspace(int batch, int H, int D, int m) {
  const int64_t pairs = static_cast<int64_t>(batch) * H;
  if (pairs >= kHilsSplitPairs) return 0;
  const size_t n = static_cast<size_t>(pairs) * m;
  return align256(n * D * 4) + align256(n * 4);
}

hipError_t launch_hils(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks, const uint16_t* v,
                       Str3 vs, const float* khat, const int32_t* chunk_idx, int batch, int L,
                       int H, int D, int C, int n_rows, int m, float scale_chunk,
                       float scale_token, uint16_t* out, Str3 os, void* ws, hipStream_t s) {
  const int pairs = batch * H;
  if (ws != nullptr && hils_workspace(batch, H, D, m) > 0) {
    const size_t n = static_cast<size_t>(pairs) * m;
    float* ws_a = static_cast<float*>(ws);
    float* ws_r = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(n * D * 4));
    const dim3 grid(pairs, (m + 3) / 4);
    if (D == 64) {
      hipLaunchKernelGGL(hils_chunks_kernel<64>, grid, dim3(256), 0, s, q, qs, k, ks, v, vs,
                         khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, ws_a,
                         ws_r);
      hipLaunchKernelGGL(hils_merge_kernel<64>, dim3(pairs), dim3(64), 0, s, ws_a, ws_r, H, m,
                         out, os);
    } else {
      hipLaunchKernelGGL(hils_chunks_kernel<128>, grid, dim3(256), 0, s, q, qs, k, ks, v, vs,
                         khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, ws_a,
                         ws_r);
      hipLaunchKernelGGL(hils_merge_kernel<128>, dim3(pairs), dim3(128), 0, s, ws_a, ws_r, H, m,
                         out, os);
    }
    return hipGetLastError();
  }
  dim3 grid(pairs);
  if (D == 64)
    hipLaunchKernelGGL((hils_kernel<64, 16>), grid, dim3(64 * 16), 0, s, q, qs, k, ks, v, vs,
                       khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  else
    hipLaunchKernelGGL((hils_kernel<128, 8>), grid, dim3(64 * 8), 0, s, q, qs, k, ks, v, vs,
                       khat, chunk_idx, L, H, C, n_rows, m, scale_chunk, scale_token, out, os);
  return hipGetLastError();
}

}  // namespace hisa
