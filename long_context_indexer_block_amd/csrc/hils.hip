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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// Bucketed prefill. Many queries share each chunk, so rather than every
// query gathering its chosen chunks, the (query, slot) entries of chunk_idx
// are bucketed by (sequence*head, chunk) and each chunk's K and V rows are
// read once per tile of 64 entries:
//   1. local keys: kloc[bh][j] = proj @ (mean of tokens j/C*C .. j), every j
//      of the chunks that hold a query of the call;
//   2. per tile, on matrix cores: the chunk's token softmax for the tile's
//      queries (causal within the local chunk) times V, normalised, into
//      partial[e][:] (scaled fp16), and the chunk logit (scale_chunk * q . key) into
//      logit[e], key = khat of the chunk or kloc of the query's position when
//      it is the query's local chunk;
//   3. per query, the softmax over its chosen chunks' logits mixes the
//      partials.
// ---------------------------------------------------------------------------
struct PrefillWs {
  PairBuckets pb;
  uint32_t* need;   // [batch][n_rows]: a query of the call lies in the chunk
  float* kloc;      // [batch*H][L][D]
  float* logit;        // [batch*H*nq*m]
  int8_t* pexp;        // [batch*H*nq*m] scale exponent of each partial row
  uint16_t* partial;   // [batch*H*nq*m][D] fp16, row scaled by 2^-pexp
};

static PrefillWs carve_prefill(void* ws, int batch, int nq, int L, int H, int D, int C, int m,
                               size_t* bytes) {
  const int bh = batch * H, nblk = (L + C - 1) / C;
  const size_t npairs = static_cast<size_t>(bh) * nq * m;
  size_t off = 0;
  PrefillWs w;
  w.pb = carve_pair_buckets(ws, bh, nq, m, nblk, &off);
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t n) { char* r = p ? p + off : nullptr; off += align256(n); return r; };
  w.need = reinterpret_cast<uint32_t*>(take(static_cast<size_t>(batch) * nblk * 4));
  w.kloc = reinterpret_cast<float*>(take(static_cast<size_t>(bh) * L * D * 4));
  w.logit = reinterpret_cast<float*>(take(npairs * 4));
  w.pexp = reinterpret_cast<int8_t*>(take(npairs));
  w.partial = reinterpret_cast<uint16_t*>(take(npairs * D * 2));
  if (bytes) *bytes = off;
  return w;
}

size_t hils_prefill_workspace(int batch, int nq, int L, int H, int D, int C, int m) {
  size_t bytes = 0;
  carve_prefill(nullptr, batch, nq, L, H, D, C, m, &bytes);
  return bytes;
}

// The chunks that hold a query of the call: only their local keys are read.
__global__ void hils_need_clear_kernel(uint32_t* __restrict__ need, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) need[i] = 0u;
}
__global__ void hils_need_mark_kernel(const int32_t* __restrict__ q_pos, int batch, int nq, int L,
                                      int C, int n_rows, uint32_t* __restrict__ need) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(batch) * nq) return;
  const int b = static_cast<int>(i / nq);
  const int t = min(max(q_pos[i], 0), L - 1);
  need[static_cast<int64_t>(b) * n_rows + t / C] = 1u;
}

// Workgroup (chunk c, pair bh): 64-token groups of the chunk; chunks that
// hold no query of the call (need[b][c] == 0) are skipped. Thread (rg, d)
// sums column d over its rows of the group (a prefix within them), the row
// groups are joined with the running carry, then thread (jg, e) projects the
// prefixes of rows jg, jg + RG, ... onto output column e.
template <int D>
__global__ __launch_bounds__(256) void hils_local_keys_kernel(
    const uint16_t* __restrict__ k, Str3 ks, int H, int L, int C,
    const uint16_t* __restrict__ proj, const uint32_t* __restrict__ need,
    float* __restrict__ kloc) {
  constexpr int RG = 256 / D;      // row groups of the scan
  constexpr int RPG = 64 / RG;     // rows per group
  __shared__ float pre[64][D];
  __shared__ float tot[RG][D];
  __shared__ float carry[D];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  if (need[static_cast<int64_t>(b) * gridDim.x + c] == 0u) return;
  const int tid = threadIdx.x, d = tid % D, rg = tid / D;
  const uint16_t* kb = k + b * ks.b + h * ks.h;
  float* out = kloc + static_cast<int64_t>(bh) * L * D;
  if (tid < D) carry[tid] = 0.0f;
  const int j_end = min(L, (c + 1) * C);
  for (int g0 = c * C; g0 < j_end; g0 += 64) {
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int j = g0 + rg * RPG + i;
      run += j < j_end ? bf16_to_f32(kb[static_cast<int64_t>(j) * ks.t + d]) : 0.0f;
      pre[rg * RPG + i][d] = run;
    }
    tot[rg][d] = run;
    __syncthreads();
    float base = carry[d];
    for (int r = 0; r < rg; ++r) base += tot[r][d];
#pragma unroll
    for (int i = 0; i < RPG; ++i) pre[rg * RPG + i][d] += base;
    __syncthreads();
    if (tid < D) {
      float all = carry[tid];
      for (int r = 0; r < RG; ++r) all += tot[r][tid];
      carry[tid] = all;
    }
    // rows jg + RG*i of the group; column e = d of this thread
    constexpr int NJ = 64 / RG;
    float acc[NJ];
    if (proj == nullptr) {
#pragma unroll
      for (int i = 0; i < NJ; ++i) acc[i] = pre[rg + RG * i][d];
    } else {
#pragma unroll
      for (int i = 0; i < NJ; ++i) acc[i] = 0.0f;
      const uint16_t* wr = proj + d * D;
      for (int x = 0; x < D; x += 8) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wr + x);
        const float wf[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                             bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
#pragma unroll
        for (int i = 0; i < NJ; ++i) {
          const float* pr = &pre[rg + RG * i][x];
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[i] = fmaf(wf[u], pr[u], acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      const int j = g0 + rg + RG * i;
      if (j < j_end)
        out[static_cast<int64_t>(j) * D + d] = acc[i] / static_cast<float>(j - c * C + 1);
    }
    __syncthreads();
  }
}

// Tile kernel: a workgroup of 4 waves takes TPW consecutive tiles of the
// tile table (mostly of one bucket, whose chunk K/V it loads once); wave w
// takes entries 16w .. 16w+15 of each tile, one per lane column r = l%16.
// The chunk's V rows are staged in LDS (rows padded by 16 bytes); so are its
// K rows when the chunk is one 64-token group (the four waves' fragments then
// come from LDS and stay in registers across tiles: K read from global once
// per workgroup instead of once per wave, 64K 6.07 -> 5.78 ms); longer
// chunks read K fragments from global per group. S^T = K Q^T on 16x16x32 bf16 MFMA leaves
// in lane l the entry l%16 and the tokens 4(l/16)..+3 of each 16-token tile:
// with the next tile's, the A operand of a 16x16x32 P V product over two
// tiles, with V^T fragments from ds_read_tr16_b64. Online softmax over the chunk's 64-token groups. Each
// wave's 16 result rows are staged in LDS and written as whole rows.
struct TileTabs {
  const uint32_t* cnt;
  const uint32_t* offs;
  const uint32_t* tile_off;
  const uint32_t* total;
  const uint32_t* pairs;
  const uint32_t* tiles;
};

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s_t;

__device__ __forceinline__ float max_x4_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_x4_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// maximum over the 16 lanes of each DPP row (every lane gets it): rotations
// by 1, 2, 4 and 8 within the row
__device__ __forceinline__ float row16_max(float v) {
  auto rot = [](float x, auto ctrl) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(__float_as_uint(x)), decltype(ctrl)::value, 0xf, 0xf, false)));
  };
  v = fmaxf(v, rot(v, std::integral_constant<int, 0x121>{}));  // row_ror:1
  v = fmaxf(v, rot(v, std::integral_constant<int, 0x122>{}));  // row_ror:2
  v = fmaxf(v, rot(v, std::integral_constant<int, 0x124>{}));  // row_ror:4
  v = fmaxf(v, rot(v, std::integral_constant<int, 0x128>{}));  // row_ror:8
  return v;
}

template <int D>
__device__ __forceinline__ void load_kfrags(uint4 (&kf)[4][D / 32], const uint16_t* kb, int64_t kst,
                                            int j0, int L, int r, int g) {
#pragma unroll
  for (int tau = 0; tau < 4; ++tau) {
    const int j = min(j0 + 16 * tau + r, L - 1);
#pragma unroll
    for (int x = 0; x < D / 32; ++x)
      kf[tau][x] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(j) * kst + 32 * x +
                                                   8 * g);
  }
}

template <int D, int C, int TPW>
__global__ __launch_bounds__(256) void hils_pair_chunk_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, const float* __restrict__ khat,
    const float* __restrict__ kloc, const int32_t* __restrict__ q_pos, int H, int nq, int L,
    int n_rows, int m, TileTabs tt, unsigned grid_wg, float scale_chunk, float scale_token_log2,
    uint16_t* __restrict__ partial, int8_t* __restrict__ pexp, float* __restrict__ logit) {
  constexpr int NKS = D / 32;     // k-steps of S^T
  constexpr int NDB = D / 16;     // 16-column blocks of O
  constexpr int NG = C / 64;      // 64-token groups per chunk
  constexpr int RS = 2 * D + 16;  // LDS bytes per staged V row
  constexpr int OS = D + 4;       // LDS floats per staged result row
  constexpr int LPR = D / 4;      // lanes per result row on the way out
  constexpr int RPI = 64 / LPR;   // result rows per store instruction
  __shared__ __align__(16) unsigned char vt[C * RS];
  __shared__ __align__(16) unsigned char kt[NG == 1 ? 64 * RS : 16];
  __shared__ __align__(16) float ot[4][16 * OS];
  // the chip deals workgroups round-robin to its 8 XCDs: give each XCD a
  // contiguous run of tiles, so that the tiles of one chunk share an L2
  const unsigned per = grid_wg / 8;
  const unsigned wg = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const unsigned ntiles = tt.total[1];
  const unsigned t_first = wg * TPW;
  if (t_first >= ntiles) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, r = l & 15;
  float* orow = ot[w];
  // ---- gathers of all TPW tiles first, so that their dependent loads
  // (tile -> bucket -> entry -> query row, position -> key row) overlap
  uint32_t key[TPW], e[TPW];
  int t[TPW];
  bool pv[TPW];
  bf16x8 qf[TPW][NKS];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
    key[j] = t_first + j < ntiles ? tt.tiles[t_first + j] : 0xffffffffu;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    pv[j] = false;
    e[j] = 0u;
    if (key[j] != 0xffffffffu) {
      const uint32_t first = tt.offs[key[j]] + (t_first + j - tt.tile_off[key[j]]) * kPairTile;
      const uint32_t pi = first + 16 * w + r;
      pv[j] = pi < tt.offs[key[j]] + tt.cnt[key[j]];
      e[j] = pv[j] ? tt.pairs[pi] : 0u;
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int bhj = static_cast<int>(key[j] / n_rows);
    const int bj = bhj / H, hj = bhj % H;
    const int qi = pv[j] ? static_cast<int>(e[j] / m - static_cast<uint32_t>(bhj) * nq) : 0;
    const uint16_t* qrow = q + bj * qs.b + static_cast<int64_t>(qi) * qs.t + hj * qs.h;
#pragma unroll
    for (int x = 0; x < NKS; ++x)
      qf[j][x] = as_bf16x8(pv[j] ? *reinterpret_cast<const uint4*>(qrow + 32 * x + 8 * g)
                                 : make_uint4(0u, 0u, 0u, 0u));
    t[j] = pv[j] ? min(max(q_pos[static_cast<int64_t>(bj) * nq + qi], 0), L - 1) : 0;
  }
  // chunk logits: q . key over this lane's columns 32x + 8g .. +7, key = the
  // chunk's khat row or, for the query's own chunk, its causal local key
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int bhj = static_cast<int>(key[j] / n_rows), cj = static_cast<int>(key[j] % n_rows);
    const int btj = t[j] / C;
    const float* kr = cj == btj ? kloc + (static_cast<int64_t>(bhj) * L + t[j]) * D
                                : khat + (static_cast<int64_t>(bhj) * n_rows + cj) * D;
    float part = 0.0f;
    if (pv[j]) {
#pragma unroll
      for (int x = 0; x < NKS; ++x) {
        const float4 k0 = *reinterpret_cast<const float4*>(kr + 32 * x + 8 * g);
        const float4 k1 = *reinterpret_cast<const float4*>(kr + 32 * x + 8 * g + 4);
        const uint4 qw = __builtin_bit_cast(uint4, qf[j][x]);
        part = fmaf(bf16_lo(qw.x), k0.x, part); part = fmaf(bf16_hi(qw.x), k0.y, part);
        part = fmaf(bf16_lo(qw.y), k0.z, part); part = fmaf(bf16_hi(qw.y), k0.w, part);
        part = fmaf(bf16_lo(qw.z), k1.x, part); part = fmaf(bf16_hi(qw.z), k1.y, part);
        part = fmaf(bf16_lo(qw.w), k1.z, part); part = fmaf(bf16_hi(qw.w), k1.w, part);
      }
    }
    part = sum_x4_groups(part);
    if (pv[j] && g == 0) logit[e[j]] = cj <= btj ? part * scale_chunk : -INFINITY;
  }
  // ---- the tiles
  uint32_t cur = 0xffffffffu;
  uint4 kf[4][NKS];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    if (key[j] == 0xffffffffu) break;
    const int bh = static_cast<int>(key[j] / n_rows), c = static_cast<int>(key[j] % n_rows);
    const int b = bh / H, h = bh % H;
    const uint16_t* kb = k + b * ks.b + h * ks.h;
    if (key[j] != cur) {
      if (cur != 0xffffffffu) __syncthreads();  // the previous chunk's V reads are done
      cur = key[j];
      const uint16_t* vb = v + b * vs.b + h * vs.h;
      for (int x = threadIdx.x; x < C * D / 8; x += 256) {
        const int row = x / (D / 8), ch = x % (D / 8);
        const int jj = min(c * C + row, L - 1);
        *reinterpret_cast<uint4*>(vt + row * RS + 16 * ch) =
            *reinterpret_cast<const uint4*>(vb + static_cast<int64_t>(jj) * vs.t + 8 * ch);
        if constexpr (NG == 1)
          *reinterpret_cast<uint4*>(kt + row * RS + 16 * ch) =
              *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(jj) * ks.t + 8 * ch);
      }
      __syncthreads();  // V (and K) staged
      if constexpr (NG == 1) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
          for (int x = 0; x < NKS; ++x)
            kf[tau][x] = *reinterpret_cast<const uint4*>(kt + (16 * tau + r) * RS + 64 * x + 16 * g);
      }
    }
    float mrun = -INFINITY, lsum = 0.0f;
    f32x4 o[NDB];
#pragma unroll
    for (int x = 0; x < NDB; ++x) o[x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int j0 = c * C + 64 * gi;
      if (j0 >= L) break;
      if constexpr (NG > 1) load_kfrags<D>(kf, kb, ks.t, j0, L, r, g);
      float sv[4][4];
      float gmax = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int x = 0; x < NKS; ++x) sacc = mfma16(as_bf16x8(kf[tau][x]), qf[j][x], sacc);
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
          const int jj = j0 + 16 * tau + 4 * g + ee;
          sv[tau][ee] = pv[j] && jj <= t[j] ? sacc[ee] * scale_token_log2 : -INFINITY;
          gmax = fmaxf(gmax, sv[tau][ee]);
        }
      }
      gmax = max_x4_groups(gmax);
      const float mnew = fmaxf(mrun, gmax);
      if (gi > 0) {
        const float alpha = mrun == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mrun - mnew);
        lsum *= alpha;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
          const float ae = __shfl(alpha, 4 * g + ee, 64);
#pragma unroll
          for (int x = 0; x < NDB; ++x) o[x][ee] *= ae;
        }
      }
      mrun = mnew;
      const float moff = mnew == -INFINITY ? 0.0f : -mnew;
      // P V for two 16-token tiles at a time: 16x16x32 products whose 8 k
      // values per lane are its 4 tokens of each tile (in P and V^T alike)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        v4s_t pa[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            const float p = __builtin_amdgcn_exp2f(sv[2 * tp + h2][ee] + moff);
            lsum += p;
            pa[h2][ee] = static_cast<short>(f32_to_bf16(p));
          }
        }
        const bf16x8 p8 =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(pa[0], pa[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const unsigned char* vrow0 =
            vt + (64 * gi + 32 * tp + 4 * g + (r >> 2)) * RS + 8 * (r & 3);
        const unsigned char* vrow1 = vrow0 + 16 * RS;
#pragma unroll
        for (int x = 0; x < NDB; ++x) {
          const v4s_t vf0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s_t*)(vrow0 + 32 * x));
          const v4s_t vf1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s_t*)(vrow1 + 32 * x));
          o[x] = mfma16(p8, __builtin_bit_cast(bf16x8, __builtin_shufflevector(vf0, vf1, 0, 1, 2, 3, 4, 5, 6, 7)),
                        o[x]);
        }
      }
    }
    lsum = sum_x4_groups(lsum);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    // O row 4g + ee (the entry of lane 4g + ee), column 16x + r -> LDS, then
    // each result row leaves as LPR 16-byte pieces
#pragma unroll
    for (int ee = 0; ee < 4; ++ee)
#pragma unroll
      for (int x = 0; x < NDB; ++x) orow[(4 * g + ee) * OS + 16 * x + r] = o[x][ee];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
    for (int it = 0; it < 16 / RPI; ++it) {
      const int rr = RPI * it + l / LPR;
      const uint32_t er = __shfl(e[j], rr, 64);
      const float ir = __shfl(inv, rr, 64);
      const int vr = __shfl(pv[j] ? 1 : 0, rr, 64);
      const float4 val = *reinterpret_cast<const float4*>(orow + rr * OS + 4 * (l % LPR));
      const float x0 = val.x * ir, x1 = val.y * ir, x2 = val.z * ir, x3 = val.w * ir;
      // the row leaves as fp16 scaled by 2^-E, E the exponent of its largest
      // magnitude (so that it lies in [0.5, 1)): 11 significant bits relative
      // to the row maximum for any magnitude; E goes to pexp
      float amax = row16_max(fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
      if constexpr (LPR == 32) amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      const int ex = min(max(static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 126, -125),
                         126);
      const float sc = __uint_as_float(static_cast<uint32_t>(127 - ex) << 23);
      if (vr) {
        const _Float16 h0 = static_cast<_Float16>(x0 * sc), h1 = static_cast<_Float16>(x1 * sc);
        const _Float16 h2 = static_cast<_Float16>(x2 * sc), h3 = static_cast<_Float16>(x3 * sc);
        const uint32_t p01 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
        const uint32_t p23 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h2)) |
                             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h3)) << 16);
        *reinterpret_cast<uint2*>(partial + static_cast<int64_t>(er) * D + 4 * (l % LPR)) =
            make_uint2(p01, p23);
        if (l % LPR == 0) pexp[er] = static_cast<int8_t>(ex);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
}

// One wave per (bh, query): the softmax over the chosen chunks' logits
// (lane s holds slot s) mixes the scaled fp16 partials. Lane l reads eight
// columns 8(l % LPS) .. +7 (16 bytes) of slots s = SL*i + l / LPS, LPS = D/8
// lanes per partial row, SL = 64/LPS slots per load instruction, four loads
// in flight; the SL lane groups are summed at the end with lane swaps.
template <int D>
__global__ __launch_bounds__(256) void hils_prefill_combine_kernel(
    const int32_t* __restrict__ chunk_idx, const int32_t* __restrict__ q_pos, int H, int nq,
    int L, int C, int m, const uint16_t* __restrict__ partial, const int8_t* __restrict__ pexp,
    const float* __restrict__ logit, uint16_t* __restrict__ out, Str3 os, int64_t nitems) {
  constexpr int LPS = D / 8;       // lanes per partial row
  constexpr int SL = 64 / LPS;     // slots per load instruction
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= nitems) return;
  const int l = threadIdx.x & 63;
  const int bh = static_cast<int>(item / nq), qi = static_cast<int>(item % nq);
  const int b = bh / H, h = bh % H;
  const int t = min(max(q_pos[static_cast<int64_t>(b) * nq + qi], 0), L - 1);
  const int bt = t / C;
  const int64_t e0 = item * m;
  const int c = l < m ? chunk_idx[e0 + l] : -1;
  const bool ok = c >= 0 && c <= bt;
  const float lg = ok ? logit[e0 + l] : -INFINITY;
  const float mx = wave_max(lg);
  const float wgt = ok && mx != -INFINITY ? __expf(lg - mx) : 0.0f;
  const float z = wave_sum(wgt);
  // the mixing weight carries the slot's partial scale 2^E
  const float wmix = ok ? wgt * __uint_as_float(static_cast<uint32_t>(127 + pexp[e0 + l]) << 23)
                        : 0.0f;
  const int sg = l / LPS, col = 8 * (l % LPS);
  float a[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) a[x] = 0.0f;
  for (int s0 = 0; s0 < m; s0 += 4 * SL) {
    uint4 val[4];
    float ws[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + SL * u + sg;
      ws[u] = __shfl(wmix, s & 63, 64);
      ws[u] = s < m ? ws[u] : 0.0f;
      val[u] = ws[u] != 0.0f ? *reinterpret_cast<const uint4*>(partial + (e0 + s) * D + col)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t wv[4] = {val[u].x, val[u].y, val[u].z, val[u].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const _Float16 h0 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(wv[x] & 0xffffu));
        const _Float16 h1 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(wv[x] >> 16));
        a[2 * x] = fmaf(ws[u], static_cast<float>(h0), a[2 * x]);
        a[2 * x + 1] = fmaf(ws[u], static_cast<float>(h1), a[2 * x + 1]);
      }
    }
  }
  // sum the SL slot groups: lanes 8 apart within a row (width 64), then the
  // four rows of 16 lanes
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    float v = a[x];
    if constexpr (LPS == 8)
      v += __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
          0, static_cast<int>(__float_as_uint(v)), 0x128, 0xf, 0xf, false)));  // row_ror:8
    a[x] = sum_x4_groups(v);
  }
  const float iz = z > 0.0f ? 1.0f / z : 0.0f;
  if (sg == 0) {
    uint16_t* orow = out + b * os.b + static_cast<int64_t>(qi) * os.t + h * os.h;
    *reinterpret_cast<uint4*>(orow + col) =
        make_uint4(pack_bf16x2(a[0] * iz, a[1] * iz), pack_bf16x2(a[2] * iz, a[3] * iz),
                   pack_bf16x2(a[4] * iz, a[5] * iz), pack_bf16x2(a[6] * iz, a[7] * iz));
  }
}

hipError_t launch_hils_prefill(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                               const uint16_t* v, Str3 vs, const float* khat,
                               const int32_t* chunk_idx, const uint16_t* proj,
                               const int32_t* q_pos, int batch, int nq, int L, int H, int D,
                               int C, int n_rows, int m, float scale_chunk, float scale_token,
                               uint16_t* out, Str3 os, void* ws, hipStream_t s) {
  if (ws == nullptr) {
    const dim3 grid(nq, batch * H);
    if (D == 64)
      hipLaunchKernelGGL((hils_prefill_kernel<64, 16>), grid, dim3(64 * 16), 0, s, q, qs, k, ks,
                         v, vs, khat, chunk_idx, proj, q_pos, nq, L, H, C, n_rows, m, scale_chunk,
                         scale_token, out, os);
    else
      hipLaunchKernelGGL((hils_prefill_kernel<128, 8>), grid, dim3(64 * 8), 0, s, q, qs, k, ks,
                         v, vs, khat, chunk_idx, proj, q_pos, nq, L, H, C, n_rows, m, scale_chunk,
                         scale_token, out, os);
    return hipGetLastError();
  }
  const int bh = batch * H;
  PrefillWs w = carve_prefill(ws, batch, nq, L, H, D, C, m, nullptr);
  hipError_t err = launch_pair_buckets(chunk_idx, bh, nq, m, n_rows, w.pb, s);
  if (err != hipSuccess) return err;
  const int nneed = batch * n_rows;
  hipLaunchKernelGGL(hils_need_clear_kernel, dim3((nneed + 255) / 256), dim3(256), 0, s, w.need,
                     nneed);
  const int64_t nqb = static_cast<int64_t>(batch) * nq;
  hipLaunchKernelGGL(hils_need_mark_kernel, dim3(static_cast<unsigned>((nqb + 255) / 256)),
                     dim3(256), 0, s, q_pos, batch, nq, L, C, n_rows, w.need);
  if (D == 64)
    hipLaunchKernelGGL((hils_local_keys_kernel<64>), dim3(n_rows, bh), dim3(256), 0, s, k, ks, H,
                       L, C, proj, w.need, w.kloc);
  else
    hipLaunchKernelGGL((hils_local_keys_kernel<128>), dim3(n_rows, bh), dim3(256), 0, s, k, ks, H,
                       L, C, proj, w.need, w.kloc);
  const size_t npairs = static_cast<size_t>(bh) * nq * m;
  const size_t max_tiles = (npairs + kPairTile - 1) / kPairTile + static_cast<size_t>(bh) * n_rows;
  // tiles per workgroup (64K at width 64: 1, 2, 4, 6, 8 tiles took 6.22,
  // 5.78, 5.59, 5.79, 5.75 ms; width 128 keeps 2 for its registers)
  const int tpw = D == 64 ? 4 : 2;
  const unsigned grid_wg = static_cast<unsigned>(((max_tiles + tpw - 1) / tpw + 7) / 8 * 8);
  const TileTabs tt{w.pb.cnt, w.pb.offs, w.pb.tile_off, w.pb.total, w.pb.pairs, w.pb.tiles};
  const float stl2 = scale_token * 1.4426950408889634f;
#define HISA_PC(D_, C_)                                                                          \
  hipLaunchKernelGGL((hils_pair_chunk_kernel<D_, C_, D_ == 64 ? 4 : 2>), dim3(grid_wg),           \
                     dim3(256), 0, s, q,                                                          \
                     qs, k, ks, v, vs, khat, w.kloc, q_pos, H, nq, L, n_rows, m, tt, grid_wg,     \
                     scale_chunk, stl2, w.partial, w.pexp, w.logit)
  if (D == 64) {
    if (C == 64) HISA_PC(64, 64); else if (C == 128) HISA_PC(64, 128); else HISA_PC(64, 256);
  } else {
    if (C == 64) HISA_PC(128, 64); else if (C == 128) HISA_PC(128, 128); else HISA_PC(128, 256);
  }
#undef HISA_PC
  const int64_t nitems = static_cast<int64_t>(bh) * nq;
  const dim3 cg(static_cast<unsigned>((nitems + 3) / 4));
  if (D == 64)
    hipLaunchKernelGGL((hils_prefill_combine_kernel<64>), cg, dim3(256), 0, s, chunk_idx, q_pos,
                       H, nq, L, C, m, w.partial, w.pexp, w.logit, out, os, nitems);
  else
    hipLaunchKernelGGL((hils_prefill_combine_kernel<128>), cg, dim3(256), 0, s, chunk_idx, q_pos,
                       H, nq, L, C, m, w.partial, w.pexp, w.logit, out, os, nitems);
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
// The same arithmetic as hils_mix, in the same order, without its chain of
// dependent loads: lane ci holds chunk ci's logit (m <= 64), read by every
// wave at once, and the partials are loaded eight chunks at a time.
template <int D>
__global__ __launch_bounds__(D) void hils_merge_kernel(const float* __restrict__ ws_a,
                                                       const float* __restrict__ ws_r, int H,
                                                       int m, uint16_t* __restrict__ out,
                                                       Str3 os) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int64_t base = static_cast<int64_t>(bh) * m;
  const int e = threadIdx.x, lane = lane_id();
  const float lg = lane < m ? ws_r[base + lane] : -INFINITY;
  const float mx = wave_max(lg);
  const float* ac = ws_a + base * D + e;
  float z = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < m; c0 += 8) {
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = c0 + j < m ? ac[(c0 + j) * D] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ci = c0 + j;
      if (ci < m) {
        const float l = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lg), ci));
        if (l != -INFINITY) {
          const float w = __expf(l - mx);
          z += w;
          acc = fmaf(w, a[j], acc);
        }
      }
    }
  }
  out[b * os.b + h * os.h + e] = f32_to_bf16(z > 0.0f ? acc / z : 0.0f);
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
